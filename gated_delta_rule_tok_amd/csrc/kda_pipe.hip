// kda_pipe.hip -- KDA chunked-prefill forward for gfx950 on 16-token chunks,
// with the state-independent work of each chunk produced ahead of the serial
// state pass by other waves of the same workgroup.
//
// The method is the bounded-gate, normalised-q/k delta rule of vLLM PR
// #55737's report ("Features and motivation"):
//   S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale S_t^T q_t,
// with log a_t = lower_bound * sigmoid(exp(A_log) (g_t + dt_bias)), b_t =
// sigmoid(beta logit) and q, k L2-normalised.  Unrolled over a chunk with G the
// inclusive cumulative log-decay (per key channel) and S the state entering it:
//   A[t,i] = b_t sum_c k_t[c] k_i[c] e^{G_t[c]-G_i[c]}        (i < t)
//   M[t,i] = scale sum_c q_t[c] k_i[c] e^{G_t[c]-G_i[c]}       (i <= t)
//   N = (I + A)^-1 diag(b) (V - (e^G k) S)
//   O = scale (e^G q) S + M N
//   S <- Diag(e^{G_last}) S + (e^{G_last - G} k)^T N
//
// Work split.  One workgroup per (sequence, head, value slice).  Eight
// "producer" waves build the packages of four 16-token chunk slots in LDS, two
// per chunk (one per 64-channel half): first the norms, the gate, the
// cumulative decay and the decayed operands of their channels, then, once the
// other half's operands are in LDS, one forms the 16x16 products A, A^T and
// the inverse (I + A)^-1, the other M.  None of it depends on the state.  The
// remaining waves ("state waves", one or two 16-column strips of the value
// slice each) walk the chunks in order, keeping their strip of S (128 x 16
// fp32) in registers, and apply the three state contractions and the output.
// There is no workgroup barrier in the main loops: each chunk slot has two
// package buffers (alternate rounds of four chunks) and LDS counters --
// producer halves that formed their operands, producer halves that finished
// their package part per buffer, the rounds each state wave is done with
// (read as one 16-byte row) -- so every
// wave waits only for the package or buffer it needs next, and the serial
// state chain, the inverse's latency chain and the next round's operand work
// overlap on each SIMD (each runs the two VALU-heavy producer waves of one
// chunk slot and one MFMA-heavy state wave).
//
// Norms.  k is normalised before it enters any product (k~ = k / ||k||, the
// norm from a dot-product pass over the row); q's norm is applied after the
// products, as a row scaling.  With rqs = scale / ||q||:
//   A[t,i] = b_t (X K_G^T)[t,i],  M'[t,i] = rqs_t (Q_T K_G^T)[t,i]
//   D = V - X S,  N = diag(b) D + L D
//   O = rqs (Q_T S) + M' N,  S <- Diag(e^{G_last}) S + K'^T N
// with X = e^G k~, Q_T = e^G q, K_G = e^{-G} k~, K' = e^{G_last - G} k~ and
// L = ((I + A)^-1 - I) diag(b).
//
// Exponent ranges.  G is taken from the chunk start, so X and K' are at most
// 1 and Q_T at most |q|, while K_G = e^{-G} k~ grows up to
// 2^{16 |lower_bound| log2 e}.  With lower_bound >= kPipeLowerBoundMin (-5)
// that is 2^115.4, inside the bf16/fp32 range.  Products of pairs t < i
// (discarded) may overflow; they are dropped by selects, not by
// multiplication.  Stronger lower bounds are served by the 64-token kernel.
//
// Precision (checked against the fp64 recurrence on the workloads'
// distributions): bf16 MFMA operands with fp32 accumulation; the inverse by
// MFMA doubling on the 16x16 block; the unit diagonal of (I + A)^-1 diag(b)
// applied in fp32.  The state update K'^T N takes fp16 operands: 16 K' (at
// most 16) and N / 16 (both scalings exact), so |N| up to 2^20 stays inside
// fp16's range, values below 2^-10 lose relative precision only down to an
// absolute 2^-21 |K'| per term, and fp16's 11-bit significand keeps each
// chunk's rounding of the fp32 state near 2^-12 of the update.
#include "kda_pipe_parts.h"

namespace kda {
namespace {

constexpr int kPW = 4;    // chunks per round
constexpr int kProdWaves = kPW * kPH;

template <int VS>
struct Cfg {
  static constexpr int NS = VS / 16;             // 16-column strips in the slice
  static constexpr int NSW = NS < 4 ? NS : 4;    // state waves
  static constexpr int SPW = NS / NSW;           // strips per state wave
  static constexpr int kThreads = 64 * (kProdWaves + NSW);
};

// Per chunk slot: per state wave the rounds it is done with (a state wave
// may run rounds ahead of another, so a shared count would not say that all
// of them left a buffer; one 16-byte row, read at once), producer-half syncs
// (counted over the run; both waves of a slot make the same sequence of
// them), and per package buffer the producer halves' finished package parts
// (both halves add one per round on that buffer).  All start at zero.
struct Sync {
  int done[kPW][4];
  int half[kPW];
  int rdy[2][kPW];
  int err;  // a bounded wait gave up
};

template <int NSW, int SPW>
struct Smem {
  Pack pk[2][kPW];              // first: keeps the packages' alignment
  bf16 kg[2][kPW][128 * kTok];  // K_G, with the package buffers, swizzled rows
  Tiles t[NSW][SPW];
  Sync sy;
};

// SUMM: the summary step of the segment-parallel schedule (p.seg_mode 1;
// see Params::seg): slices over 256 columns, the transition half with zero
// values from the identity, no outputs.
template <int VS, bool SUMM>
__global__ __launch_bounds__(Cfg<VS>::kThreads, 1) void pipe_kernel(Params p) {
  using C = Cfg<VS>;
  constexpr int SPW = C::SPW, NSW = C::NSW;
  __shared__ __attribute__((aligned(16))) Smem<NSW, SPW> sm;
  Pack (&pk)[2][kPW] = sm.pk;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a uniform (scalar) value: the two roles below run separate
  // loops, each with one barrier per round
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (sequence rank, head, slice): ranks in order across the XCDs,
  // the slices of one head on one XCD (sharing q/k/g in its L2)
  const int b = work_item(blockIdx.x, gridDim.x, p.vsplit);
  const int slice = b % p.vsplit;
  const int rest = b / p.vsplit;
  const int h = rest % p.H;
  const int H = p.H;
  // sequence of rank rest / H (longest first, ties by index): from the plan
  // table, or ranked here when there are few sequences
  if (tid < int(sizeof(Sync) / sizeof(int))) reinterpret_cast<int*>(&sm.sy)[tid] = 0;
  int n, m = 0;  // sequence; pseudo-sequence (segment) of the segment-parallel schedule
  int4 segent = {0, 0, 0, 1};
  if (p.seg) {
    m = rest / H;
    segent = reinterpret_cast<const int4*>(p.seg)[m];
    n = __builtin_amdgcn_readfirstlane(segent.x);
    // unused entries, and last segments in the summary step, have nothing to
    // do (the whole workgroup leaves: n and the flags are uniform)
    if (n < 0 || (SUMM && (__builtin_amdgcn_readfirstlane(segent.w) & 1))) return;
  } else if (p.order) {
    n = p.order[rest / H];
  } else {
    // scratch in a package that nothing uses yet (no other LDS allocation, so
    // the packages keep their alignment)
    int* seq_sh = reinterpret_cast<int*>(pk[1][kPW - 1].gam);
    const int N = p.N, target = rest / H;
    if (tid <= N) seq_sh[tid] = p.cu[tid];
    __syncthreads();
    int len = 0, rank = 0;
    if (tid < N) {
      len = seq_sh[tid + 1] - seq_sh[tid];
      for (int m = 0; m < N; ++m) {
        const int lm = seq_sh[m + 1] - seq_sh[m];
        rank += (lm > len) || (lm == len && m < tid);
      }
    }
    __syncthreads();
    if (tid < N && rank == target) seq_sh[0] = tid;
    __syncthreads();
    // uniform by construction; as a scalar, every address and buffer
    // resource derived from it stays in scalar registers
    n = __builtin_amdgcn_readfirstlane(seq_sh[0]);
  }
  __syncthreads();  // counters zeroed, ranking scratch read: the packages are free

  // the bounds are uniform: scalar registers (else every buffer access with a
  // token offset in its scalar operand becomes a loop over lanes)
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.seg ? segent.y : p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.seg ? segent.z : p.cu[n + 1], bos), p.T));
  const bool seg_last = (__builtin_amdgcn_readfirstlane(segent.w) & 1) != 0;
  const int nc = (eos - bos + kTok - 1) / kTok;  // chunks
  const int nr = (nc + kPW - 1) / kPW;            // rounds

  // ---------------- producer waves ----------------
  // wave = chunk slot c of the round + kPW * channel half hf; the two waves
  // of a chunk share a SIMD.  One instance per half (hf known at compile
  // time: the first half loads no q rows, the second no beta, with no
  // branch around the loads)
  auto producer = [&](auto half) {
    constexpr int hf = decltype(half)::value;
    const int c = wave & (kPW - 1);
    RawSrc src;
    // (the summary step forms no output: no q, its loads read zeros)
    src.q = rows_rsrc(p.q + size_t(h) * p.hs_q, SUMM ? 0 : eos, p.ts_q, kD);
    src.k = rows_rsrc(p.k + size_t(h) * p.hs_k, eos, p.ts_k, kD);
    src.g = rows_rsrc(p.g + size_t(h) * p.hs_g, eos, p.ts_g, kD);
    src.qn = rows_rsrc(p.q + size_t(h) * p.hs_q, hf && !SUMM ? eos : 0, p.ts_q, kD);
    src.beta = rows_rsrc(p.beta + size_t(h) * p.hs_b, hf ? 0 : eos, p.ts_b, 1);
    const float eA = expf(p.A_log[h]);
    const float c1 = -kLog2e * eA;
    const float lb2 = p.lower_bound * kLog2e;
    float c2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c2[i] = c1 * p.dt_bias[h * kD + 64 * hf + 4 * (lane & 15) + i];
    __builtin_amdgcn_sched_barrier(0);  // constants first: nothing waits behind the first chunk's loads
    const RawLoad ld{src, p.ts_q, p.ts_k, p.ts_g, p.ts_b, lane, hf};
    Raw raw;
    ld.all(raw, bos + kTok * c);
    for (int r = 0; r < nr; ++r) {
      const int j = kPW * r + c;
      if (j >= nc) break;
      Pack& P = pk[r & 1][c];
      bf16* kg = sm.kg[r & 1][c];
      // the buffers are free once every state wave is done with round r - 2
      if (r >= 2)
        wait_row<NSW>(sm.sy.done[c], r - 1, &sm.sy.err);
      const int t0 = bos + kTok * j, Lc = min(kTok, eos - t0);
      // this wave's next chunk (one round ahead) is loaded while the operands
      // are formed
      const int tn = t0 + kTok * kPW;
      // one code path for full and partial chunks: with two, the registers
      // of the next chunk's loads differ between them and the merge copies
      // them, which waits for the loads at the end of every round
      produce_operands<false, SUMM>(P, kg, raw, ld, tn, hf, Lc, lane, c2, c1, lb2, p.scale);
      // both halves' operands (the products run over all 128 channels)
      arrive(&sm.sy.half[c], lane);
      wait_count(&sm.sy.half[c], kPH * (r + 1), &sm.sy.err);
      if (hf == 0) produce_inverse(P, kg, lane);
      else if (!SUMM) produce_m(P, kg, lane);
      arrive(&sm.sy.rdy[r & 1][c], lane);
    }
  };
  if (wave < kProdWaves) {
    if (wave < kPW) producer(BufIdx<0>{});
    else producer(BufIdx<1>{});
    if (lane == 0 && gave_up(&sm.sy.err)) p.errword[0] = 1;
    return;
  }

  // ---------------- state waves ----------------
  // The state waves carry the serial chain; give them issue priority over the
  // producer wave that shares their SIMD.
  __builtin_amdgcn_s_setprio(2);
  // S[u][rt][j] = S[16 rt + 4 g4 + j][column of strip u]
  const int sw = wave - kProdWaves;
  // summary step: slices 0 .. vsplit/2 - 1 carry the local state, the others
  // the transition, whose values are zero (an empty range: its loads read
  // zeros without touching memory)
  const bool trans = SUMM && slice >= p.vsplit / 2;
  const int vslice = trans ? slice - p.vsplit / 2 : slice;
  const int colb = vslice * VS + 16 * sw + l16;  // column of strip 0; strip u adds 16 NSW u
  const __amdgpu_buffer_rsrc_t vsrc = rows_rsrc(p.v + size_t(h) * p.hs_v, trans ? 0 : eos, p.ts_v, kD);
  const __amdgpu_buffer_rsrc_t odst = rows_rsrc(p.out + size_t(h) * p.hs_o, eos, p.ts_o, kD);
  // the state's [D, D] block: sequence n's, or in the segment-parallel
  // schedule the segment's (summary: local state, then transition)
  const size_t sbase = (size_t(n) * H + h) * kD * kD;
  const size_t segbase = SUMM ? ((size_t(m) * H + h) * 2 + (trans ? 1 : 0)) * kD * kD
                              : (size_t(m) * H + h) * kD * kD;
  f32x4 S[SPW][8];
  // this wave's strips of the state, in the state dtype, into the [D, D]
  // block at dst + base
  auto store_state = [&](void* dst, size_t base) {
    if (p.state_bf16) {
#pragma unroll
      for (int u = 0; u < SPW; ++u)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            static_cast<bf16*>(dst)[base + size_t(16 * rt + 4 * g4 + j) * kD + colb + 16 * NSW * u] =
                (bf16)S[u][rt][j];
    } else {
#pragma unroll
      for (int u = 0; u < SPW; ++u)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            static_cast<float*>(dst)[base + size_t(16 * rt + 4 * g4 + j) * kD + colb + 16 * NSW * u] =
                S[u][rt][j];
    }
  };
  // checkpoint states: the first slot of this sequence (the checkpoints of
  // the sequences before it, summed over the lanes), the chunk count of the
  // next checkpoint and its slot
  int ck_slot = 0, ck_next = 0, ck_chunks = 0;
  if (p.ck) {
    int acc = 0;
    for (int m = lane; m < n; m += 64) {
      const int b0 = min(max(p.cu[m], 0), p.T);
      const int e0 = min(max(p.cu[m + 1], b0), p.T);
      acc += (e0 - b0) / p.ck_int;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    ck_slot = __builtin_amdgcn_readfirstlane(acc);
    ck_chunks = p.ck_int / kTok;
    ck_next = ck_chunks;
  }
  if (SUMM) {
    // local state from zero, transition from the identity
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S[u][rt][j] = trans && 16 * rt + 4 * g4 + j == colb + 16 * NSW * u ? 1.f : 0.f;
  } else if (!p.s0) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (p.seg) {
    // a segment's entering state (fp32, from the combine step)
    const float* s0 = static_cast<const float*>(p.s0) + segbase + colb;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][rt][j] = s0[(16 * rt + 4 * g4 + j) * kD + 16 * NSW * u];
  } else if (p.state_bf16) {
    const uint16_t* s0 = static_cast<const uint16_t*>(p.s0) + sbase + colb;
    uint16_t raw0[SPW][8][4];
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) raw0[u][rt][j] = s0[(16 * rt + 4 * g4 + j) * kD + 16 * NSW * u];
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][rt][j] = bf16_to_f32(raw0[u][rt][j]);
  } else {
    const float* s0 = static_cast<const float*>(p.s0) + sbase + colb;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][rt][j] = s0[(16 * rt + 4 * g4 + j) * kD + 16 * NSW * u];
  }
  // values of each round's chunks, loaded one round before use into two
  // alternating register sets (no copies, so nothing waits for the output
  // stores issued in between)
  const unsigned cstrip = unsigned(vslice * VS + 16 * sw);  // first column of strip 0
  uint2 va[kPW][SPW], vbuf[kPW][SPW];
#pragma unroll
  for (int c = 0; c < kPW; ++c)
#pragma unroll
    for (int u = 0; u < SPW; ++u) va[c][u] = vbuf[c][u] = uint2{0u, 0u};

  // Unconditional: chunks past the sequence end read as zeros (range check);
  // conditional loads would make the compiler wait for every outstanding
  // memory operation (output stores included) before each load.
  auto load_round = [&](uint2 (&v)[kPW][SPW], int r) {
#pragma unroll
    for (int c = 0; c < kPW; ++c) {
      const int t0 = bos + kTok * (kPW * r + c);
#pragma unroll
      for (int u = 0; u < SPW; ++u) v[c][u] = load_vrow(vsrc, cstrip + 16 * NSW * u, p.ts_v, t0, lane);
    }
  };
  // chunks of round r, in order, from package buffer B = r % 2, each once
  // its producers are done with it (compile-time indices, so every LDS read
  // is a lane offset plus a constant)
  auto consume_round = [&](const uint2 (&v)[kPW][SPW], int r, auto buf) {
    constexpr int B = decltype(buf)::value;
#pragma unroll
    for (int c = 0; c < kPW; ++c) {
      const int j = kPW * r + c;
      if (j >= nc) break;
      // both halves of the package: rounds B, B + 2, .., r on this buffer
      wait_count(&sm.sy.rdy[B][c], kPH * ((r >> 1) + 1), &sm.sy.err);
      const Pack& P = pk[B][c];
      const int t0 = bos + kTok * j;

      // X and Q_T as A operands; k-slots {32kb + 4g4 + j, 32kb + 16 + 4g4 + j}
      // match the B operand built from two accumulator tiles of S
      bf16x8 ax[4], aq[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const int r1 = 32 * kb2 + 4 * g4 + (l16 >> 2), r2 = r1 + 16;
        const int o1 = tile(r1, l16 & 3), o2 = tile(r2, l16 & 3);
        ax[kb2] = cat(tr4(&P.x[o1]), tr4(&P.x[o2]));
        if constexpr (!SUMM) aq[kb2] = cat(tr4(&P.qt[o1]), tr4(&P.qt[o2]));
      }
      const f32x4 bR = *reinterpret_cast<const f32x4*>(&P.beta[4 * g4]);
      const f32x4 rqR = *reinterpret_cast<const f32x4*>(&P.rqs[4 * g4]);
      const bf16x4 Lf = *reinterpret_cast<const bf16x4*>(&P.l[frag(0, l16, 4 * g4)]);
      const bf16x4 Mf = *reinterpret_cast<const bf16x4*>(&P.m[frag(0, l16, 4 * g4)]);
      // V in the accumulator layout (it does not depend on S, so it is formed
      // before the chain): the row tile read back transposed (lane l16 of
      // group g4: column l16 of tokens 4 g4 .. 4 g4 + 3); this wave's own LDS
      // accesses are processed in order
      f32x4 V[SPW];
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        Tiles& tl = sm.t[sw][u];
        *reinterpret_cast<uint2*>(&tl.v[4 * lane]) = v[c][u];
        __builtin_amdgcn_wave_barrier();
        V[u] = to_f32x4(tr4(&tl.v[4 * lane]));
      }

#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        bf16x8 Sb[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
          Sb[kb2] = cat(to_bf16x4(S[u][2 * kb2]), to_bf16x4(S[u][2 * kb2 + 1]));
        f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
          Y = mfma32(ax[kb2], Sb[kb2], Y);
          if constexpr (!SUMM) Q = mfma32(aq[kb2], Sb[kb2], Q);  // (output only)
        }
        // the products are issued here; the decay Diag(e^{G_last}) of the
        // state (its bf16 copy is already taken) is applied while they run,
        // before their results are used (a wave issues in order, so anything
        // placed after that point would lengthen the chain to the update)
        asm volatile("" : "+v"(Y), "+v"(Q));
        {
          const float2 gv = *reinterpret_cast<const float2*>(&P.gam[16 * (l16 >> 1) + 4 * g4 + 2 * (l16 & 1)]);
          decay_strip(S[u], gv.x, gv.y);
        }
        asm volatile("" : "+v"(S[u][0]), "+v"(S[u][1]), "+v"(S[u][2]), "+v"(S[u][3]),
                     "+v"(S[u][4]), "+v"(S[u][5]), "+v"(S[u][6]), "+v"(S[u][7]), "+v"(Y), "+v"(Q));
        Tiles& tl = sm.t[sw][u];
        const f32x4 D = V[u] - Y;
        const f32x4 N = mfma16(Lf, to_bf16x4(D), bR * D);
        if constexpr (!SUMM) {  // (the summary step writes no output)
          const f32x4 O = mfma16(Mf, to_bf16x4(N), rqR * Q);
          // O into rows: written column-major, read back transposed (lane l16
          // of group g4: columns 4 g4 .. + 3 of token l16), one 8-byte store
          // per lane; rows past the sequence end are dropped by the range check
          *reinterpret_cast<uint2*>(&tl.o[16 * l16 + 4 * g4]) = uint2{pk2(O[0], O[1]), pk2(O[2], O[3])};
          __builtin_amdgcn_wave_barrier();
          const bf16x4 orow = tr4(&tl.o[64 * g4 + 16 * (l16 >> 2) + 4 * (l16 & 3)]);
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(u32x2, orow), odst,
              ((unsigned(t0) + unsigned(l16)) * unsigned(p.ts_o) + cstrip + 16 * NSW * u + 4u * g4) * 2u,
              0, 0);
        }
        // S <- (Diag(e^{G_last}) S) + K'^T N in fp16 operands (kKpScale K' and
        // kNScale N; k-slots: this lane group's four tokens).  The accumulator
        // comes from the VALU (the decay above), never straight from a product
        // of another MFMA shape: on gfx950 a 16x16x16 product accumulating onto
        // a 16x16x32 result was observed to return wrong sums.
        const f16x4 Nq = f16x4{(_Float16)(N[0] * kNScale), (_Float16)(N[1] * kNScale),
                               (_Float16)(N[2] * kNScale), (_Float16)(N[3] * kNScale)};
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
          const f16x4 a = *reinterpret_cast<const f16x4*>(&P.kp[fragx(rt, l16, 4 * g4)]);
          S[u][rt] = mfma16h(a, Nq, S[u][rt]);
        }
      }
      arrive(&sm.sy.done[c][sw], lane);
      // the state after the first (j + 1) chunks, when that is a checkpoint
      // (whole chunks only: a sequence's last, partial chunk never ends on
      // a multiple of the interval)
      if (p.ck && j + 1 == ck_next && kTok * (j + 1) <= eos - bos) {
        if (ck_slot < p.ck_cap) store_state(p.ck, (size_t(ck_slot) * H + h) * kD * kD);
        ++ck_slot;
        ck_next += ck_chunks;
      }
    }
  };

  load_round(va, 0);
  for (int r = 0; r < nr; r += 2) {  // r even: buffer 0; r + 1: buffer 1
    load_round(vbuf, r + 1);
    consume_round(va, r, BufIdx<0>{});
    if (r + 1 < nr) {
      load_round(va, r + 2);
      consume_round(vbuf, r + 1, BufIdx<1>{});
    }
  }

  // final state: the sequence's (or, in the segment-parallel schedule, its
  // last segment's), or the summary of a segment
  if (SUMM) store_state(p.sT, segbase);
  else if (seg_last) store_state(p.sT, sbase);
  if (lane == 0 && gave_up(&sm.sy.err)) p.errword[0] = 1;
}

}  // namespace

hipError_t launch_pipe(const Params& p, hipStream_t stream) {
  const void* fn = nullptr;
  int threads = 0;
  if (p.seg_mode == 1) {  // summaries: 4 slices of 64 over 256 columns
    if (p.vsplit != 4 || !p.seg) return hipErrorInvalidValue;
    fn = reinterpret_cast<const void*>(&pipe_kernel<64, true>);
    threads = Cfg<64>::kThreads;
  } else {
    switch (kD / p.vsplit) {
      case 64: fn = reinterpret_cast<const void*>(&pipe_kernel<64, false>); threads = Cfg<64>::kThreads; break;
      case 32: fn = reinterpret_cast<const void*>(&pipe_kernel<32, false>); threads = Cfg<32>::kThreads; break;
      case 16: fn = reinterpret_cast<const void*>(&pipe_kernel<16, false>); threads = Cfg<16>::kThreads; break;
      default: return hipErrorInvalidValue;
    }
  }
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(p.N * p.H * p.vsplit), dim3(threads), args, 0, stream);
}

}  // namespace kda
