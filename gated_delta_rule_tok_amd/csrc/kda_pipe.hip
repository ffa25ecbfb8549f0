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
// Work split.  One workgroup per (sequence, head, value slice).  Waves 0-3
// ("producers") each take every fourth 16-token chunk and build the chunk's
// package in LDS: the gate, the cumulative decay, the decayed operands, the
// 16x16 products A and M, the inverse (I + A)^-1, and the norms.  None of it
// depends on the state.  The remaining waves ("state waves", one or two
// 16-column strips of the value slice each) walk the chunks in order, keeping
// their strip of S (128 x 16 fp32) in registers, and apply the three state
// contractions and the output.  Packages are double-buffered per round of
// four chunks: in round r the producers write round r while the state waves
// read round r-1; one workgroup barrier ends each round.  On gfx950 this puts
// a VALU-heavy producer wave and an MFMA-heavy state wave on every SIMD.
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
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kTok = 16;  // tokens per chunk
constexpr int kPW = 4;    // producer waves = chunks per round
constexpr float kKpScale = 16.f;     // K' enters the fp16 state update times this
constexpr float kNScale = 0.0625f;   // ... and N times this (exact inverse)

template <int VS>
struct Cfg {
  static constexpr int NS = VS / 16;             // 16-column strips in the slice
  static constexpr int NSW = NS < 4 ? NS : 4;    // state waves
  static constexpr int SPW = NS / NSW;           // strips per state wave
  static constexpr int kThreads = 64 * (kPW + NSW);
};

// [128][16] tiles (row = key channel, column = token): rows are stored in the
// order swz(r), which keeps both the producers' 16-byte row writes (8 lanes
// write rows 4c + i, c = 0..3, two halves each) and the transposed operand
// reads (4 consecutive rows x 32 bytes) on distinct banks.
__device__ __forceinline__ int swz(int r) { return r ^ ((r >> 2) & 3); }

// Fragment tiles: the A-operand order of a 16x16x16 MFMA.  Element (row m,
// column k) of 16x16 block b sits at (b * 64) + ((k / 4) * 16 + m) * 4 + k % 4,
// so lane (l16, g4) reads its four k-values as 8 contiguous bytes and a wave
// reads one block as 512 contiguous bytes.
__device__ __forceinline__ int frag(int blk, int m, int k) {
  return blk * 256 + ((k >> 2) * 16 + m) * 4 + (k & 3);
}

// Buffer resources over one head's rows of a [T, H, ...] tensor, bounded at
// the end of the sequence: loads past it return 0 and stores past it are
// dropped by the hardware range check, so partial chunks need no branches.
// (gfx9 buffer descriptor word 3: 32-bit untyped data.)
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int eos, int rowstride,
                                                          int rowlen) {
  const int bytes = eos > 0 ? ((eos - 1) * rowstride + rowlen) * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

template <int B>
struct BufIdx {
  static constexpr int value = B;
};

// One chunk's package: written by one producer wave, read by the state waves.
struct Pack {
  bf16 x[128 * kTok];    // X = e^{G} k~, swizzled rows
  bf16 qt[128 * kTok];   // Q_T = e^{G} q, swizzled rows
  bf16 kp[128 * kTok];   // kKpScale K' as fp16, fragment order (block = 16 keys);
                         // before that, scratch for K_G (bf16, swizzled rows)
  bf16 l[256];           // L, fragment order
  bf16 m[256];           // M', fragment order
  float beta[kTok];
  float rk[kTok];        // 1 / ||k_t|| (producer scratch)
  float rqs[kTok];       // scale / ||q_t||
  float gam[128];        // e^{G_last}
};
static_assert(sizeof(Pack::gam) >= sizeof(int) * (kInlineRankMax + 1), "rank scratch fits in gam");

// Raw inputs of one chunk for one producer lane: tokens 8 th + rr of channels
// 4 cg .. 4 cg + 3 (cg = lane / 2, th = lane % 2); q and k again as rows for
// the norms (token lane / 4, channels 32 (lane % 4) ..); the beta logit of
// token `lane` (lanes < 16).
struct Raw {
  uint2 q[8], k[8], g[8];
  uint4 qn[4], kn[4];
  uint32_t beta;
};

struct RawSrc {
  __amdgpu_buffer_rsrc_t q, k, g, beta;  // head h, bounded at the sequence end
};

// Rows past the sequence end read as zeros (buffer range check).
__device__ __forceinline__ void load_raw(Raw& r, const RawSrc& src, int rowstride, int H, int t0,
                                         int lane) {
  const unsigned ch = 4u * unsigned(lane >> 1), th = unsigned(lane & 1);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const unsigned off = ((unsigned(t0) + 8u * th + rr) * unsigned(rowstride) + ch) * 2u;
    r.q[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.q, off, 0, 0));
    r.k[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.k, off, 0, 0));
    r.g[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.g, off, 0, 0));
  }
  const unsigned offn =
      ((unsigned(t0) + unsigned(lane >> 2)) * unsigned(rowstride) + 32u * unsigned(lane & 3)) * 2u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.qn[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src.q, offn + 16u * i, 0, 0));
    r.kn[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src.k, offn + 16u * i, 0, 0));
  }
  r.beta = __builtin_amdgcn_raw_buffer_load_b16(src.beta, (unsigned(t0) + unsigned(lane)) * unsigned(H) * 2u, 0, 0);
}

__device__ __forceinline__ float dot2(uint32_t a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, a), c, false);
}

__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}

__device__ __forceinline__ uint32_t pk2h(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
}

// Sum over the four lanes 4 i .. 4 i + 3.
__device__ __forceinline__ float quad_sum(float s) {
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
  return s;
}

// Channel i (0..3) of a 4-channel bf16 group.
__device__ __forceinline__ float chan(uint2 w, int i) {
  const uint32_t d = i < 2 ? w.x : w.y;
  return (i & 1) ? bf16_hi(d) : bf16_lo(d);
}

// Values a producer keeps in registers across its MFMA step: kKpScale K' as
// packed fp16 pairs of consecutive tokens, per channel.
struct Held {
  uint32_t kp[4][4];
};

// Producer, first half: norms of q and k, beta, the gate and its cumulative
// sum, and every decayed operand.  Writes X = e^G k~ and Q_T = e^G q (which
// are also the left operands of the A and M products), the scratch right
// operand K_G = e^{-G} k~, gam, beta and rqs; returns K' in `held`.  FULL:
// all 16 tokens are inside the sequence (no masking).
template <bool FULL>
__device__ __forceinline__ void produce_operands(Pack& pk, const Raw& raw, Held& held, int Lc,
                                                 int lane, const float* c2, float c1, float lb2,
                                                 float scale) {
  const int cg = lane >> 1, th = lane & 1;

  // scale / ||q_t|| and 1 / ||k_t|| for token lane/4: four lanes hold 32
  // channels each
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sq = dot2(raw.qn[i].x, sq);
      sq = dot2(raw.qn[i].y, sq);
      sq = dot2(raw.qn[i].z, sq);
      sq = dot2(raw.qn[i].w, sq);
      sk = dot2(raw.kn[i].x, sk);
      sk = dot2(raw.kn[i].y, sk);
      sk = dot2(raw.kn[i].z, sk);
      sk = dot2(raw.kn[i].w, sk);
    }
    sq = quad_sum(sq);
    sk = quad_sum(sk);
    if ((lane & 3) == 0) {
      pk.rqs[lane >> 2] = rsqrtf(sq + kNormEps) * scale;
      pk.rk[lane >> 2] = rsqrtf(sk + kNormEps);
    }
    if (lane < kTok)
      pk.beta[lane] = lane < Lc ? rcp(1.f + ex2(-kLog2e * bf16_to_f32(uint16_t(raw.beta)))) : 0.f;
  }

  // gate sigma per (token, channel) and its running sum over this lane's 8
  // tokens; the log2 decay of a token is lb2 * sigma (lb2 = lower_bound log2 e)
  float cs[4][8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const bool valid = FULL || 8 * th + rr < Lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sg = rcp(1.f + ex2(fmaf(chan(raw.g[rr], i), c1, c2[i])));
      const float inc = valid ? sg : 0.f;
      cs[i][rr] = rr == 0 ? inc : cs[i][rr - 1] + inc;
    }
  }

  // G relative to the chunk start.  Lane th = 0 holds tokens 0..7, lane
  // th = 1 tokens 8..15 and adds the partner's total of tokens 0..7.
  float off[4], gam[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float own = cs[i][7], other = pair_swap(own);
    off[i] = th ? lb2 * other : 0.f;
    gam[i] = ex2(lb2 * (own + other));  // e^{G_last}
  }
  if (th == 0) *reinterpret_cast<f32x4*>(&pk.gam[4 * cg]) = f32x4{gam[0], gam[1], gam[2], gam[3]};

  // 1 / ||k|| of this lane's 8 tokens (written above by other lanes of this wave)
  __builtin_amdgcn_wave_barrier();
  const f32x4 rk0 = *reinterpret_cast<const f32x4*>(&pk.rk[8 * th]);
  const f32x4 rk1 = *reinterpret_cast<const f32x4*>(&pk.rk[8 * th + 4]);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = swz(4 * cg + i) * kTok + 8 * th;  // this lane's 8 tokens of channel 4cg+i
    const float g16 = kKpScale * gam[i];
    uint32_t xk[4], qk[4], kg[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      float vx[2], vq[2], vg[2], vkp[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rr = 2 * pr + h;
        const float G = fmaf(cs[i][rr], lb2, off[i]);
        const float E = ex2(G), F = ex2(-G);
        const float kv = chan(raw.k[rr], i) * (rr < 4 ? rk0[rr] : rk1[rr - 4]);
        const float qv = chan(raw.q[rr], i);
        vx[h] = kv * E;
        vq[h] = qv * E;
        vg[h] = kv * F;
        vkp[h] = vg[h] * g16;
      }
      xk[pr] = pk2(vx[0], vx[1]);
      qk[pr] = pk2(vq[0], vq[1]);
      kg[pr] = pk2(vg[0], vg[1]);
      held.kp[i][pr] = pk2h(vkp[0], vkp[1]);
    }
    *reinterpret_cast<uint4*>(&pk.x[row]) = uint4{xk[0], xk[1], xk[2], xk[3]};
    *reinterpret_cast<uint4*>(&pk.qt[row]) = uint4{qk[0], qk[1], qk[2], qk[3]};
    *reinterpret_cast<uint4*>(&pk.kp[row]) = uint4{kg[0], kg[1], kg[2], kg[3]};
  }
}

// Producer, second half: the A and M products, the inverse and L, then K'
// over the scratch operand (this wave's own LDS accesses are
// processed in order, so the scratch reads are done before it is
// overwritten).
__device__ __forceinline__ void produce_products(Pack& pk, const Held& held, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const int cg = lane >> 1, th = lane & 1;

  // A = X K_G^T, A^T = K_G X^T and M'^T = K_G Q_T^T over the 128 channels;
  // k-slots 8 g4 .. 8 g4 + 7 of each 32-channel block, on both sides
  __builtin_amdgcn_wave_barrier();  // the operands were written by other lanes of this wave
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 accA = zero, accAt = zero, accMt = zero;
  const int col = 4 * (l16 & 3);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int r1 = 32 * kb + 8 * g4 + (l16 >> 2), r2 = r1 + 4;
    const int o1 = swz(r1) * kTok + col, o2 = swz(r2) * kTok + col;
    const bf16x8 KE = cat(tr4(&pk.x[o1]), tr4(&pk.x[o2]));
    const bf16x8 KG = cat(tr4(&pk.kp[o1]), tr4(&pk.kp[o2]));
    const bf16x8 QE = cat(tr4(&pk.qt[o1]), tr4(&pk.qt[o2]));
    accA = mfma32(KE, KG, accA);     // [t = 4g4+j][i = l16]
    accAt = mfma32(KG, KE, accAt);   // [i = 4g4+j][t = l16]
    accMt = mfma32(KG, QE, accMt);   // [i = 4g4+j][t = l16]
  }

  // beta and rqs were written by other lanes of this wave (before the
  // operand writes that the barrier above orders)
  const f32x4 bR = *reinterpret_cast<const f32x4*>(&pk.beta[4 * g4]);
  const float bC = pk.beta[l16], rqC = pk.rqs[l16];

  f32x4 Nn, Nt, Mv, I4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g4 + j;
    Nn[j] = l16 < r ? bR[j] * accA[j] : 0.f;    // A[r][l16]
    Nt[j] = r < l16 ? bC * accAt[j] : 0.f;      // A[l16][r]
    Mv[j] = r <= l16 ? rqC * accMt[j] : 0.f;                   // M'[l16][r]
    I4[j] = r == l16 ? 1.f : 0.f;
  }
  *reinterpret_cast<bf16x4*>(&pk.m[frag(0, l16, 4 * g4)]) = to_bf16x4(Mv);

  // (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) (A^16 = 0).  Each product is
  // formed together with its transpose: an accumulator holds Z[4g+j][l16],
  // which is Z's B-operand layout and Z^T's A-operand layout, so Z = X Y is
  // mfma(X^T, Y) and Z^T = Y^T X^T is mfma(Y, X^T).
  {
    const bf16x4 nb = to_bf16x4(Nn), ntb = to_bf16x4(Nt);
    const f32x4 N2 = mfma16(ntb, nb, zero), N2t = mfma16(nb, ntb, zero);
    const bf16x4 n2b = to_bf16x4(N2), n2tb = to_bf16x4(N2t);
    const f32x4 N4 = mfma16(n2tb, n2b, zero), N4t = mfma16(n2b, n2tb, zero);
    const bf16x4 n4b = to_bf16x4(N4), n4tb = to_bf16x4(N4t);
    const f32x4 N8 = mfma16(n4tb, n4b, zero);
    const f32x4 P1t = mfma16(n2b, to_bf16x4(-Nt), I4 - Nt + N2t);   // (I - A)(I + A^2)
    const bf16x4 p1tb = to_bf16x4(P1t);
    const f32x4 P2t = mfma16(n4b, p1tb, P1t);                        // ... (I + A^4)
    const bf16x4 p2tb = to_bf16x4(P2t), n8b = to_bf16x4(N8);
    const f32x4 Dt = mfma16(n8b, p2tb, P2t);                         // D^T: D[l16][4g4+j]
    // L[t][i] = (D - I)[t][i] b_i at fragment (m = t = l16, k = i = 4g4 + j)
    *reinterpret_cast<bf16x4*>(&pk.l[frag(0, l16, 4 * g4)]) = to_bf16x4((Dt - I4) * bR);
  }

  // K' over K_G (this wave's scratch reads above come first in its LDS order)
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * cg + i;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int o = frag(c >> 4, c & 15, 8 * th + 4 * hh);
      *reinterpret_cast<uint2*>(&pk.kp[o]) = uint2{held.kp[i][2 * hh], held.kp[i][2 * hh + 1]};
    }
  }
}

// Value strip of one chunk for a state lane: tokens 4 g4 + j of one column,
// one register each, raw bf16 bits (zero past the sequence end).  Nothing
// combines the values here, so nothing waits for these loads before the
// chunk that uses them.
__device__ __forceinline__ void load_v4(uint32_t* e, __amdgpu_buffer_rsrc_t v, unsigned col,
                                        int rowstride, int t0, int g4) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    e[j] = __builtin_amdgcn_raw_buffer_load_b16(
        v, ((unsigned(t0) + unsigned(4 * g4 + j)) * unsigned(rowstride) + col) * 2u, 0, 0);
}

template <int VS>
__global__ __launch_bounds__(Cfg<VS>::kThreads, 1) void pipe_kernel(Params p) {
  using C = Cfg<VS>;
  constexpr int SPW = C::SPW, NSW = C::NSW;
  __shared__ __attribute__((aligned(16))) Pack pk[2][kPW];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a uniform (scalar) value: the two roles below run separate
  // loops, each with one barrier per round
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (sequence rank, head, slice); the slices of one head stay on
  // one XCD so they share q/k/g in its L2
  int b = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int slice = b % p.vsplit;
  const int rest = b / p.vsplit;
  const int h = rest % p.H;
  const int H = p.H;
  // sequence of rank rest / H (longest first, ties by index): from the plan
  // table, or ranked here when there are few sequences
  int n;
  if (p.order) {
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


  const int bos = min(max(p.cu[n], 0), p.T);
  const int eos = min(max(p.cu[n + 1], bos), p.T);
  const int nc = (eos - bos + kTok - 1) / kTok;  // chunks
  const int nr = (nc + kPW - 1) / kPW;            // rounds
  const int rowstride = H * kD;

  if (wave < kPW) {
    // ---------------- producer waves ----------------
    RawSrc src;
    src.q = rows_rsrc(p.q + size_t(h) * kD, eos, rowstride, kD);
    src.k = rows_rsrc(p.k + size_t(h) * kD, eos, rowstride, kD);
    src.g = rows_rsrc(p.g + size_t(h) * kD, eos, rowstride, kD);
    src.beta = rows_rsrc(p.beta + h, eos, H, 1);
    const float eA = expf(p.A_log[h]);
    const float c1 = -kLog2e * eA;
    const float lb2 = p.lower_bound * kLog2e;
    float c2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c2[i] = c1 * p.dt_bias[h * kD + 4 * (lane >> 1) + i];
    __builtin_amdgcn_sched_barrier(0);  // constants first: nothing waits behind the first chunk's loads
    Raw raw;
    if (wave < nc) load_raw(raw, src, rowstride, H, bos + kTok * wave, lane);
    for (int r = 0; r <= nr; ++r) {
      const int j = kPW * r + wave;
      if (r < nr && j < nc) {
        const int t0 = bos + kTok * j, Lc = min(kTok, eos - t0);
        Pack& P = pk[r & 1][wave];
        Held held;
        if (Lc == kTok) produce_operands<true>(P, raw, held, Lc, lane, c2, c1, lb2, p.scale);
        else produce_operands<false>(P, raw, held, Lc, lane, c2, c1, lb2, p.scale);
        // this wave's next chunk, one round ahead
        const int tn = t0 + kTok * kPW;
        if (tn < eos) load_raw(raw, src, rowstride, H, tn, lane);
        produce_products(P, held, lane);
      }
      __syncthreads();
    }
    return;
  }

  // ---------------- state waves ----------------
  // The state waves carry the serial chain; give them issue priority over the
  // producer wave that shares their SIMD.
  __builtin_amdgcn_s_setprio(2);
  // S[u][rt][j] = S[16 rt + 4 g4 + j][column of strip u]
  const int sw = wave - kPW;
  const int colb = slice * VS + 16 * sw + l16;  // column of strip 0; strip u adds 16 NSW u
  const __amdgpu_buffer_rsrc_t vsrc = rows_rsrc(p.v + size_t(h) * kD, eos, rowstride, kD);
  const __amdgpu_buffer_rsrc_t odst = rows_rsrc(p.out + size_t(h) * kD, eos, rowstride, kD);
  const size_t sbase = (size_t(n) * H + h) * kD * kD;
  f32x4 S[SPW][8];
  if (!p.s0) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
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
  uint32_t va[kPW][SPW][4], vbuf[kPW][SPW][4];
#pragma unroll
  for (int c = 0; c < kPW; ++c)
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) va[c][u][j] = vbuf[c][u][j] = 0u;

  auto load_round = [&](uint32_t (&v)[kPW][SPW][4], int r) {
    if (r >= nr) return;
#pragma unroll
    for (int c = 0; c < kPW; ++c) {
      const int t0 = bos + kTok * (kPW * r + c);
      if (t0 < eos)
#pragma unroll
        for (int u = 0; u < SPW; ++u) load_v4(v[c][u], vsrc, colb + 16 * NSW * u, rowstride, t0, g4);
    }
  };
  // the chunks of round r - 1, in order, from package buffer B = (r - 1) % 2
  // (a compile-time index, so every LDS read is a lane offset plus a constant)
  auto consume_round = [&](const uint32_t (&v)[kPW][SPW][4], int r, auto buf) {
    constexpr int B = decltype(buf)::value;
#pragma unroll
    for (int c = 0; c < kPW; ++c) {
      const int j = kPW * (r - 1) + c;
      if (j >= nc) break;
      const Pack& P = pk[B][c];
      const int t0 = bos + kTok * j;

      // X and Q_T as A operands; k-slots {32kb + 4g4 + j, 32kb + 16 + 4g4 + j}
      // match the B operand built from two accumulator tiles of S
      bf16x8 ax[4], aq[4];
      const int col = 4 * (l16 & 3);
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const int r1 = 32 * kb2 + 4 * g4 + (l16 >> 2), r2 = r1 + 16;
        const int o1 = swz(r1) * kTok + col, o2 = swz(r2) * kTok + col;
        ax[kb2] = cat(tr4(&P.x[o1]), tr4(&P.x[o2]));
        aq[kb2] = cat(tr4(&P.qt[o1]), tr4(&P.qt[o2]));
      }
      const f32x4 bR = *reinterpret_cast<const f32x4*>(&P.beta[4 * g4]);
      const f32x4 rqR = *reinterpret_cast<const f32x4*>(&P.rqs[4 * g4]);
      const bf16x4 Lf = *reinterpret_cast<const bf16x4*>(&P.l[frag(0, l16, 4 * g4)]);
      const bf16x4 Mf = *reinterpret_cast<const bf16x4*>(&P.m[frag(0, l16, 4 * g4)]);

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
          Q = mfma32(aq[kb2], Sb[kb2], Q);
        }
        f32x4 V;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) V[jj] = bf16_lo(v[c][u][jj]);
        const f32x4 D = V - Y;
        const f32x4 N = mfma16(Lf, to_bf16x4(D), bR * D);
        const f32x4 O = mfma16(Mf, to_bf16x4(N), rqR * Q);
        // rows past the sequence end are dropped by the range check (the
        // halves are taken from packed words: storing bf16 vector elements
        // directly through the 16-bit buffer store is miscompiled)
        const uint32_t w01 = pk2(O[0], O[1]), w23 = pk2(O[2], O[3]);
        const unsigned short ov[4] = {(unsigned short)w01, (unsigned short)(w01 >> 16),
                                      (unsigned short)w23, (unsigned short)(w23 >> 16)};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          __builtin_amdgcn_raw_buffer_store_b16(
              ov[jj], odst,
              ((unsigned(t0) + unsigned(4 * g4 + jj)) * unsigned(rowstride) + colb + 16 * NSW * u) * 2u,
              0, 0);
        // S <- Diag(e^{G_last}) S + K'^T N in fp16 operands (kKpScale K' and
        // kNScale N; k-slots: this lane group's four tokens).  The accumulator
        // comes from the VALU (S gm), never straight from a product of another
        // MFMA shape: on gfx950 a 16x16x16 product accumulating onto a
        // 16x16x32 result was observed to return wrong sums.
        const f16x4 Nq = f16x4{(_Float16)(N[0] * kNScale), (_Float16)(N[1] * kNScale),
                               (_Float16)(N[2] * kNScale), (_Float16)(N[3] * kNScale)};
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
          const f32x4 gm = *reinterpret_cast<const f32x4*>(&P.gam[16 * rt + 4 * g4]);
          const f16x4 a = *reinterpret_cast<const f16x4*>(&P.kp[frag(rt, l16, 4 * g4)]);
          S[u][rt] = mfma16h(a, Nq, S[u][rt] * gm);
        }
      }
    }
  };

  load_round(va, 0);
  __syncthreads();
  for (int r = 1; r <= nr; r += 2) {  // r odd: buffer 0; r + 1: buffer 1
    load_round(vbuf, r);
    consume_round(va, r, BufIdx<0>{});
    __syncthreads();
    if (r + 1 <= nr) {
      load_round(va, r + 1);
      consume_round(vbuf, r + 1, BufIdx<1>{});
      __syncthreads();
    }
  }

  // final state
#pragma unroll
  for (int u = 0; u < SPW; ++u)
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t idx = sbase + size_t(16 * rt + 4 * g4 + j) * kD + colb + 16 * NSW * u;
        if (p.state_bf16) static_cast<bf16*>(p.sT)[idx] = (bf16)S[u][rt][j];
        else static_cast<float*>(p.sT)[idx] = S[u][rt][j];
      }
}

}  // namespace

hipError_t launch_pipe(const Params& p, hipStream_t stream) {
  const void* fn = nullptr;
  int threads = 0;
  switch (kD / p.vsplit) {
    case 128: fn = reinterpret_cast<const void*>(&pipe_kernel<128>); threads = Cfg<128>::kThreads; break;
    case 64: fn = reinterpret_cast<const void*>(&pipe_kernel<64>); threads = Cfg<64>::kThreads; break;
    case 32: fn = reinterpret_cast<const void*>(&pipe_kernel<32>); threads = Cfg<32>::kThreads; break;
    case 16: fn = reinterpret_cast<const void*>(&pipe_kernel<16>); threads = Cfg<16>::kThreads; break;
    default: return hipErrorInvalidValue;
  }
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(p.N * p.H * p.vsplit), dim3(threads), args, 0, stream);
}

}  // namespace kda
