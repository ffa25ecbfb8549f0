// kda_chunk.hip -- chunked (WY / UT) KDA forward for gfx950 with bf16 MFMA.
//
// One workgroup of 4 waves per (sequence, head, value slice of VS columns)
// walks the chunks of 64 tokens of its sequence.  The state slice S
// (128 key rows x VS value columns, fp32) stays in MFMA accumulator registers
// for the whole sequence.  Per chunk, with G the inclusive cumulative
// log-decay inside the chunk (per key channel) and S the state entering it:
//
//   A[t,i] = b_t sum_c k_t[c] k_i[c] e^{G_t[c]-G_i[c]}   (i < t)
//   Mq[t,i] =   sum_c q_t[c] k_i[c] e^{G_t[c]-G_i[c]}    (i <= t; q carries scale)
//   Tm = (I + A)^-1,  L = (Tm - I) diag(b)
//   W = diag(b) (e^G k) + L (e^G k),   U = diag(b) V + L V
//   N = U - W S
//   O = (e^G q) S + Mq N
//   S <- Diag(e^{G_last}) S + (e^{G_last - G} k)^T N
//
// which is the recurrence S_t = (I - b k k^T) Diag(a_t) S_{t-1} + b k v^T,
// o_t = scale S_t^T q_t of vLLM PR #55737's report ("Features and
// motivation": bounded gate, in-kernel q/k L2 norm, raw beta logits) unrolled
// over a chunk: the pseudo-values N solve a unit lower-triangular system,
// which is the "chunk path" the page says the fused kernel replaces.
//
// Precision plan (checked against the fp64 recurrence on the workloads'
// distributions): q, k, the decays, A and Mq in bf16 MFMA with fp32
// accumulation; the triangular inverse in fp32 on its 16x16 diagonal blocks
// and bf16 MFMA across blocks; W and U keep their unit-diagonal term exact
// (b * X added in fp32), only L is bf16; the state update uses a two-term
// (hi + lo) bf16 split of both operands (three products), so the fp32 state
// does not pick up bf16 rounding each chunk.
//
// Overflow: e^{G_t - G_i} is factored as e^{G_t - R} e^{R - G_i} with the
// reference R at token 7 of each 16-token sub-chunk, so every factor inside
// a sub-chunk stays within e^{+-16|lower_bound|}; pairs of different
// sub-chunks use the later sub-chunk's reference and an extra per-channel
// factor e^{R_a - R_b} <= 1 on the earlier sub-chunk's operand.
//
// gfx950 facts used here, each checked on the device:
//  * v_mfma_f32_16x16x{32,16}_bf16: lane l holds accumulator rows 4*(l/16)+j of
//    column l%16.  Operand k-slots only have to agree between A and B, so a
//    k-block of 32 built from two accumulator tiles uses the slot order
//    {4g..4g+3, 16+4g..16+4g+3} (g = l/16) on both sides.
//  * ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
//    the 8-byte loads of lanes i/4, 4+i/4, 8+i/4, 12+i/4.  With lane L pointing
//    at row base+L/4, columns c0+4*(L%4).., lane i gets column c0+i of rows
//    base..base+3 -- an operand with k running over rows, read straight from a
//    row-major [token][channel] array.  So every operand stays row-major.
//  * v_permlane16_swap / v_permlane32_swap exchange 16-lane rows and 32-lane
//    halves; they carry the cumulative-sum scan across the rows of a wave.
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 64;  // tokens per chunk

// LDS row strides in bf16 elements, chosen for the access each array sees:
constexpr int kRowA = 136;  // 68 dwords = 4 mod 32: 16-row 16-byte operand reads
constexpr int kRowT = 144;  // 72 dwords = 8 mod 32: transpose reads (4 rows x 32 B)
constexpr int kRowW = 132;  // 66 dwords = 2 mod 32: 16-row 8-byte operand reads
constexpr int kRowM = 68;   // 64 x 64 token-token matrices read 8 bytes per row
constexpr int kRowL = 72;   // 64 x 64 read 16 bytes per row

// Sum over the 16 lanes of a DPP row (all 16 lanes get the same bits).
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// Exclusive prefix sum over the four 16-lane rows of a wave (per lane column).
__device__ __forceinline__ float rows_exclusive_sum(float x, int row) {
  const uint32_t u = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float from_prev_row = __uint_as_float(s16[0]);  // odd rows: row - 1
  const float from_next_row = __uint_as_float(s16[1]);  // even rows: row + 1
  const bool odd = row & 1;
  const float pair = x + (odd ? from_prev_row : from_next_row);  // t0+t1 or t2+t3
  const uint32_t up = __float_as_uint(pair);
  const auto s32 = __builtin_amdgcn_permlane32_swap(up, up, false, false);
  const float low_pair = __uint_as_float(s32[0]);  // rows 2, 3: t0 + t1
  return (odd ? from_prev_row : 0.f) + (row >= 2 ? low_pair : 0.f);
}

// Operand with k over 4 consecutive rows base.. and lane column c0 + l16 of a
// row-major array: the transpose read with lane L at row base + L/4.
template <int STRIDE>
__device__ __forceinline__ bf16x4 rows4(const bf16 (*arr)[STRIDE], int base, int c0, int l16) {
  return tr4(&arr[base + (l16 >> 2)][c0 + 4 * (l16 & 3)]);
}

// A-operand rows for a k-block of 32 whose B operand was built from two
// accumulator tiles: slots 0..3 <- columns base+4g.., slots 4..7 <- base+16+4g..
template <int STRIDE>
__device__ __forceinline__ bf16x8 perm_row(const bf16 (*arr)[STRIDE], int row, int base, int g4) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&arr[row][base + 4 * g4]);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&arr[row][base + 16 + 4 * g4]);
  return cat(lo, hi);
}

// Pair index -> block (a, b), b <= a, of the 4 x 4 sub-chunk blocks.
__device__ __forceinline__ void pair_ab(int pi, int& a, int& b) {
  a = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
  b = pi - (a * (a + 1)) / 2;
}

template <int VS>
struct Smem {
  static constexpr int VROW = VS + 16 > 48 ? VS + 16 : 48;  // transpose reads
  bf16 ke[kC][kRowA];   // k^ e^{G-R} (A left operand); then e^G k^ (W right operand)
  bf16 qe[kC][kRowA];   // (scale q^) e^{G-R} (Mq left); then e^G (scale q^) (O left)
  union {
    bf16 kf[kC][kRowA];  // k^ e^{R-G} (A / Mq right operand)
    struct {
      bf16 row[4][16][24];  // diagonal inverse blocks D_a, row-major
      bf16 col[4][16][24];  // the same, transposed
    } d;
    bf16 wn[kC][kRowW];  // -W
  } r2;
  bf16 kph[kC][kRowT];  // e^{G_last-G} k^, high bf16 part
  bf16 kpl[kC][kRowT];  // low part
  bf16 v[kC][VROW];     // value slice [token][column]
  float adt[4][16][20];  // diagonal blocks of A, transposed: adt[a][m][r] = A[16a+r][16a+m]
  bf16 aoff[kC][kRowM];  // off-diagonal blocks of A; then Mq
  bf16 lb[kC][kRowL];    // L = (Tm - I) diag(b)
  float beta[kC];
  float rloc[4][128];   // G at token 7 of each sub-chunk, relative to the sub-chunk start
  float wtot[4][128];   // log-decay total of each sub-chunk
  float dab[7][128];    // e^{R_a - R_b}, a > b; row 6 holds ones (diagonal blocks)
  float gam[128];       // e^{G_last}
};

// Global values of one chunk, fetched one chunk ahead.  Thread (tq, co) =
// (tid / 16, tid % 16) covers tokens 4tq..4tq+3, key channels 8co..8co+7 and
// value columns co*VN..co*VN+VN-1 of the slice.
template <int VS>
struct Prefetch {
  static constexpr int VN = VS / 16;
  uint4 q[4], k[4], g[4];
  bf16 v[4][VN];
  uint16_t beta;  // raw bits: converting here would wait for the load
};

template <int VS>
__device__ __forceinline__ void load_row(Prefetch<VS>& pf, int r, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* g, const uint16_t* v) {
  constexpr int VN = Prefetch<VS>::VN;
  pf.q[r] = *reinterpret_cast<const uint4*>(q);
  pf.k[r] = *reinterpret_cast<const uint4*>(k);
  pf.g[r] = *reinterpret_cast<const uint4*>(g);
  const bf16* vp = reinterpret_cast<const bf16*>(v);
  if constexpr (VN == 8) {
    *reinterpret_cast<bf16x8*>(pf.v[r]) = *reinterpret_cast<const bf16x8*>(vp);
  } else if constexpr (VN == 4) {
    *reinterpret_cast<bf16x4*>(pf.v[r]) = *reinterpret_cast<const bf16x4*>(vp);
  } else {
#pragma unroll
    for (int c = 0; c < VN; ++c) pf.v[r][c] = vp[c];
  }
}

// Fetch chunk [t0, t0 + L).  Offsets are 32-bit from uniform base pointers
// (q/k/g/v point at token 0 of head h; v at this slice's first column).
// Token strides (elements) of the per-token tensors.
struct TokStrides {
  unsigned q, k, g, v, b;
};

template <int VS>
__device__ __forceinline__ void load_chunk(Prefetch<VS>& pf, const uint16_t* q, const uint16_t* k,
                                           const uint16_t* g, const uint16_t* v,
                                           const uint16_t* beta, const TokStrides& ts, int t0,
                                           int L, int tq, int tid) {
  constexpr int VN = Prefetch<VS>::VN;
  const unsigned ck = 8u * (unsigned)(tid & 15), cv = (unsigned)(tid & 15) * VN;
  if (L == kC) {  // full chunk: no per-row predicates
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned t = (unsigned)(t0 + 4 * tq + r);
      load_row<VS>(pf, r, q + (t * ts.q + ck), k + (t * ts.k + ck), g + (t * ts.g + ck),
                   v + (t * ts.v + cv));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      if (t < L) {
        const unsigned tt = (unsigned)(t0 + t);
        load_row<VS>(pf, r, q + (tt * ts.q + ck), k + (tt * ts.k + ck), g + (tt * ts.g + ck),
                     v + (tt * ts.v + cv));
      } else {
        pf.q[r] = pf.k[r] = pf.g[r] = uint4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < VN; ++c) pf.v[r][c] = (bf16)0.f;
      }
    }
  }
  pf.beta = (tid < L) ? beta[(unsigned)(t0 + tid) * ts.b] : uint16_t(0);
}

// Elementwise pass of one chunk, kept in registers until the chunk's operand
// phase: raw q and k, their per-token inverse norms (q's includes scale), the
// log2 decay summed from the start of this wave's 16-token sub-chunk, and the
// raw value slice and beta logit.  Writes the sub-chunk's reference value
// (token 7) and total to LDS for the operand phase.
template <int VS>
struct Elem {
  uint4 q[4], k[4];
  float rq[4], rk[4];
  float lam[4][8];
  bf16 v[4][Prefetch<VS>::VN];
  float beta;
};

template <int VS>
__device__ __forceinline__ void elementwise(Elem<VS>& el, const Prefetch<VS>& pf, int L, int tq,
                                            int g4, const float* c2, float c1, float lb2,
                                            float scale, float* rloc_row, float* wtot_row) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float qf[8], kf[8], gf[8];
    unpack8(pf.q[r], qf);
    unpack8(pf.k[r], kf);
    unpack8(pf.g[r], gf);
    el.q[r] = pf.q[r];
    el.k[r] = pf.k[r];
#pragma unroll
    for (int c = 0; c < Prefetch<VS>::VN; ++c) el.v[r][c] = pf.v[r][c];
    float qq = 0.f, kk = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qq = fmaf(qf[i], qf[i], qq);
      kk = fmaf(kf[i], kf[i], kk);
    }
    el.rq[r] = rsqrtf(row_sum16(qq) + kNormEps) * scale;
    el.rk[r] = rsqrtf(row_sum16(kk) + kNormEps);
    const bool valid = 4 * tq + r < L;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // log2 of the decay: lb * sigmoid(exp(A_log) (g + dt_bias)) * log2(e)
      const float e = ex2(fmaf(gf[i], c1, c2[i]));
      el.lam[r][i] = valid ? lb2 * rcp(1.f + e) : 0.f;
    }
  }
  el.beta = bf16_to_f32(pf.beta);
  // inclusive cumulative sum from the start of this wave's 16-token sub-chunk
#pragma unroll
  for (int r = 1; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) el.lam[r][i] += el.lam[r - 1][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float excl = rows_exclusive_sum(el.lam[3][i], g4);
#pragma unroll
    for (int r = 0; r < 4; ++r) el.lam[r][i] += excl;
  }
  const f32x4 lo = f32x4{el.lam[3][0], el.lam[3][1], el.lam[3][2], el.lam[3][3]};
  const f32x4 hi = f32x4{el.lam[3][4], el.lam[3][5], el.lam[3][6], el.lam[3][7]};
  if (g4 == 1) {  // token 7 of the sub-chunk
    reinterpret_cast<f32x4*>(rloc_row)[0] = lo;
    reinterpret_cast<f32x4*>(rloc_row)[1] = hi;
  }
  if (g4 == 3) {  // sub-chunk total
    reinterpret_cast<f32x4*>(wtot_row)[0] = lo;
    reinterpret_cast<f32x4*>(wtot_row)[1] = hi;
  }
}

template <int VS>
__global__ __launch_bounds__(kThreads, 1) void chunk_kernel(Params p) {
  constexpr int NS = VS / 16;                // 16-column strips in the slice
  constexpr int SPW = NS >= 4 ? NS / 4 : 1;  // strips per wave
  constexpr int VN = Prefetch<VS>::VN;
  __shared__ __attribute__((aligned(16))) Smem<VS> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;  // MFMA lane coordinates
  const int tq = tid >> 4, co = tid & 15;     // elementwise coordinates (g4 = tq % 4)
  const int ch0 = 8 * co;

  // workgroup -> (sequence rank, head, slice): ranks in order across the XCDs,
  // the slices of one head on one XCD (sharing q/k/g in its L2)
  const int b = work_item(blockIdx.x, gridDim.x, p.vsplit);
  const int slice = b % p.vsplit;
  const int rest = b / p.vsplit;
  const int h = rest % p.H;
  const int n = p.order[rest / p.H];
  const int H = p.H;

  // zero the triangular buffers whose upper blocks are never written
  for (int i = tid; i < kC * kRowM / 8; i += kThreads)
    reinterpret_cast<uint4*>(&sm.aoff[0][0])[i] = uint4{0, 0, 0, 0};
  for (int i = tid; i < kC * kRowL / 8; i += kThreads)
    reinterpret_cast<uint4*>(&sm.lb[0][0])[i] = uint4{0, 0, 0, 0};

  // per-head constants: sigmoid argument and lower bound in log2 units
  const float eA = expf(p.A_log[h]);
  const float c1 = -kLog2e * eA;
  float c2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c2[i] = c1 * p.dt_bias[h * kD + ch0 + i];
  const float lb2 = p.lower_bound * kLog2e;

  // state slice in accumulator layout: S[st][rt][j] = S[16 rt + 4 g4 + j][16 s + l16]
  f32x4 S[SPW][8];
  const size_t sbase = ((size_t)n * H + h) * kD * kD;
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    const int s = wave + 4 * st;
    const int jg = slice * VS + 16 * s + l16;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = 0.f;
        if (s < NS && p.s0) {
          const size_t idx = sbase + (size_t)(16 * rt + 4 * g4 + j) * kD + jg;
          x = p.state_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.s0)[idx])
                           : static_cast<const float*>(p.s0)[idx];
        }
        S[st][rt][j] = x;
      }
  }

  // the bounds are uniform: scalar registers (else every buffer access with a
  // token offset in its scalar operand becomes a loop over lanes)
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n + 1], bos), p.T));

  // base pointers of token 0 for this head (and this thread's channels);
  // per-token offsets below are 32-bit ((T + 256) * stride < 2^31 elements is
  // checked on the host)
  const TokStrides ts{unsigned(p.ts_q), unsigned(p.ts_k), unsigned(p.ts_g), unsigned(p.ts_v),
                      unsigned(p.ts_b)};
  const unsigned ts_o = unsigned(p.ts_o);
  const uint16_t* qb = p.q + (size_t)h * p.hs_q;
  const uint16_t* kb = p.k + (size_t)h * p.hs_k;
  const uint16_t* gb = p.g + (size_t)h * p.hs_g;
  const uint16_t* vb = p.v + (size_t)h * p.hs_v + slice * VS;
  const uint16_t* betab = p.beta + (size_t)h * p.hs_b;
  uint16_t* outb = p.out + (size_t)h * p.hs_o + slice * VS;

  Prefetch<VS> pf;
  Elem<VS> el;
  if (bos < eos) {
    load_chunk<VS>(pf, qb, kb, gb, vb, betab, ts, bos, min(kC, eos - bos), tq, tid);
    elementwise<VS>(el, pf, min(kC, eos - bos), tq, g4, c2, c1, lb2, p.scale, &sm.rloc[wave][ch0],
                    &sm.wtot[wave][ch0]);
  }

  for (int t0 = bos; t0 < eos; t0 += kC) {
    const int L = min(kC, eos - t0);
    __syncthreads();  // the previous chunk is done with every shared buffer

    // fetch the next chunk; its elementwise pass runs during this chunk's state part
    const int Ln = min(kC, eos - t0 - kC);  // <= 0 when this is the last chunk
    if (Ln > 0) load_chunk<VS>(pf, qb, kb, gb, vb, betab, ts, t0 + kC, Ln, tq, tid);

    // ---------------- decay factors and MFMA operands ----------------
    // R: G at token 7 of this sub-chunk (relative to the sub-chunk start);
    // pre: G before the sub-chunk; tot: G at the chunk's last token
    float eR[8];
    {
      float R[8], eLR[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        R[i] = sm.rloc[wave][ch0 + i];
        float pre = 0.f, tot = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float wt = sm.wtot[w][ch0 + i];
          if (w < wave) pre += wt;
          tot += wt;
        }
        eR[i] = ex2(pre + R[i]);          // e^{R} from the chunk start
        eLR[i] = ex2(tot - pre - R[i]);   // e^{G_last - R}
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tq + r;
        float qf[8], kf[8], ke[8], qe[8], kfv[8], kph[8], kpl[8];
        unpack8(el.q[r], qf);
        unpack8(el.k[r], kf);
#pragma unroll
        for (int c = 0; c < VN; ++c) sm.v[t][co * VN + c] = el.v[r][c];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float E = ex2(el.lam[r][i] - R[i]);
          const float F = ex2(R[i] - el.lam[r][i]);
          const float kn = kf[i] * el.rk[r];
          kfv[i] = kn * F;
          ke[i] = kn * E;
          qe[i] = qf[i] * el.rq[r] * E;
          const float kp = kfv[i] * eLR[i];  // e^{G_last - G_t} k^
          const float hi = (float)(bf16)kp;
          kph[i] = hi;
          kpl[i] = kp - hi;
        }
        *reinterpret_cast<bf16x8*>(&sm.ke[t][ch0]) = pack8(ke);
        *reinterpret_cast<bf16x8*>(&sm.qe[t][ch0]) = pack8(qe);
        *reinterpret_cast<bf16x8*>(&sm.r2.kf[t][ch0]) = pack8(kfv);
        *reinterpret_cast<bf16x8*>(&sm.kph[t][ch0]) = pack8(kph);
        *reinterpret_cast<bf16x8*>(&sm.kpl[t][ch0]) = pack8(kpl);
      }
    }
    if (tid < kC) sm.beta[tid] = tid < L ? rcp(1.f + ex2(-kLog2e * el.beta)) : 0.f;
    for (int idx = tid; idx < 6 * 128; idx += kThreads) {
      const int pr = idx >> 7, c = idx & 127;
      const int a = pr < 1 ? 1 : pr < 3 ? 2 : 3;
      const int bb = pr - (a * (a - 1)) / 2;
      float d = sm.rloc[a][c] - sm.rloc[bb][c];
      for (int w = bb; w < a; ++w) d += sm.wtot[w][c];
      sm.dab[pr][c] = ex2(d);
    }
    if (tid < 128) sm.dab[6][tid] = 1.f;
    if (tid < 128) sm.gam[tid] = ex2(sm.wtot[0][tid] + sm.wtot[1][tid] + sm.wtot[2][tid] + sm.wtot[3][tid]);
    __syncthreads();

    // ---------------- A and Mq blocks (bf16 MFMA over the 128 channels) ----------------
    // wave w takes pairs w, w+4, w+8 of the 10 lower blocks; waves 2 and 3 repeat
    // pair 9 as a third, discarded pair so the compute stays branch-free
    f32x4 accA[3], accM[3];
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
      const int pi = min(wave + 4 * k3, 9);
      int a, bb;
      pair_ab(pi, a, bb);
      const float* drow = &sm.dab[bb < a ? (a * (a - 1)) / 2 + bb : 6][0];  // row 6: ones
      accA[k3] = accM[k3] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c0 = 32 * ks + 8 * g4;
        const bf16x8 aK = *reinterpret_cast<const bf16x8*>(&sm.ke[16 * a + l16][c0]);
        const bf16x8 aQ = *reinterpret_cast<const bf16x8*>(&sm.qe[16 * a + l16][c0]);
        const bf16x8 bK = *reinterpret_cast<const bf16x8*>(&sm.r2.kf[16 * bb + l16][c0]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(drow + c0);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(drow + c0 + 4);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = (float)bK[i] * d0[i];
          f[4 + i] = (float)bK[4 + i] * d1[i];
        }
        const bf16x8 bKd = pack8(f);
        accA[k3] = mfma32(aK, bKd, accA[k3]);
        accM[k3] = mfma32(aQ, bKd, accM[k3]);
      }
    }
    f32x4 Mreg[3];
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
      const int pi = wave + 4 * k3;
      int a, bb;
      pair_ab(min(pi, 9), a, bb);
      f32x4 at;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g4 + j;  // row inside the block
        const bool keepA = bb < a || l16 < r;
        const bool keepM = bb < a || l16 <= r;
        at[j] = keepA ? accA[k3][j] * sm.beta[16 * a + r] : 0.f;
        Mreg[k3][j] = keepM ? accM[k3][j] : 0.f;
      }
      if (pi < 10) {
        if (bb == a) {
          *reinterpret_cast<f32x4*>(&sm.adt[a][l16][4 * g4]) = at;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) sm.aoff[16 * a + 4 * g4 + j][16 * bb + l16] = (bf16)at[j];
        }
      }
    }
    __syncthreads();

    // ---------------- (I + A)^-1 on the diagonal blocks; q, k operands -> e^G ----------------
    {
      // D = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for the strictly lower
      // 16x16 block N = A_aa (N^16 = 0), one block per wave.  Every product is
      // formed together with its transpose: an accumulator holds Z[4g+j][l16],
      // which is Z's B-operand layout and Z^T's A-operand layout, so Z = X Y is
      // mfma(X^T, Y) and Z^T = Y^T X^T is mfma(Y, X^T).
      const int a = wave;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 Nn = *reinterpret_cast<const f32x4*>(&sm.adt[a][l16][4 * g4]);  // N[4g+j][l16]
      f32x4 Nt;                                                                  // N[l16][4g+j]
#pragma unroll
      for (int j = 0; j < 4; ++j) Nt[j] = sm.adt[a][4 * g4 + j][l16];
      f32x4 I4;
#pragma unroll
      for (int j = 0; j < 4; ++j) I4[j] = (4 * g4 + j == l16) ? 1.f : 0.f;
      const bf16x4 nb = to_bf16x4(Nn), ntb = to_bf16x4(Nt);
      const f32x4 N2 = mfma16(ntb, nb, zero), N2t = mfma16(nb, ntb, zero);
      const bf16x4 n2b = to_bf16x4(N2), n2tb = to_bf16x4(N2t);
      const f32x4 N4 = mfma16(n2tb, n2b, zero), N4t = mfma16(n2b, n2tb, zero);
      const bf16x4 n4b = to_bf16x4(N4), n4tb = to_bf16x4(N4t);
      const f32x4 N8 = mfma16(n4tb, n4b, zero);
      // P1 = I - N + N^2 - N N^2
      const f32x4 P1 = mfma16(ntb, to_bf16x4(-N2), I4 - Nn + N2);
      const f32x4 P1t = mfma16(n2b, to_bf16x4(-Nt), I4 - Nt + N2t);
      // P2 = P1 (I + N^4)
      const bf16x4 p1tb = to_bf16x4(P1t);
      const f32x4 P2 = mfma16(p1tb, n4b, P1);
      const f32x4 P2t = mfma16(n4b, p1tb, P1t);
      // D = P2 (I + N^8)
      const bf16x4 p2tb = to_bf16x4(P2t), n8b = to_bf16x4(N8);
      const f32x4 D = mfma16(p2tb, n8b, P2);    // D[4g+j][l16]
      const f32x4 Dt = mfma16(n8b, p2tb, P2t);  // D[l16][4g+j]
      // row-major D (A operand of D_a X), column-major D (B operand of A_ab D_b),
      // and the diagonal block of L = (D - I) diag(b)
      *reinterpret_cast<bf16x4*>(&sm.r2.d.row[a][l16][4 * g4]) = to_bf16x4(Dt);
      *reinterpret_cast<bf16x4*>(&sm.r2.d.col[a][l16][4 * g4]) = to_bf16x4(D);
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * a + 4 * g4]);
      *reinterpret_cast<bf16x4*>(&sm.lb[16 * a + l16][16 * a + 4 * g4]) = to_bf16x4((Dt - I4) * bt);
    }
    // e^G k^ (W's right operand) and e^G (scale q^) (O's left operand), in place
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(&sm.ke[t][ch0]);
      const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(&sm.qe[t][ch0]);
      float fk[8], fq[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        fk[i] = (float)k8[i] * eR[i];
        fq[i] = (float)q8[i] * eR[i];
      }
      *reinterpret_cast<bf16x8*>(&sm.ke[t][ch0]) = pack8(fk);
      *reinterpret_cast<bf16x8*>(&sm.qe[t][ch0]) = pack8(fq);
    }
    __syncthreads();

    // ---------------- off-diagonal blocks: wave b builds column b of Tm ----------------
    // T_ab = -D_a sum_{c=b}^{a-1} A_ac T_cb, with T_bb = D_b
    if (wave < 3) {
      const int bb = wave;
      bf16x4 Tc[4];  // T_cb of this column as B operands (c > b)
#pragma unroll
      for (int a = 1; a < 4; ++a) {
        if (a <= bb) continue;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c < bb || c >= a) continue;
          const bf16x4 Aop = *reinterpret_cast<const bf16x4*>(&sm.aoff[16 * a + l16][16 * c + 4 * g4]);
          const bf16x4 Bop = c == bb ? *reinterpret_cast<const bf16x4*>(&sm.r2.d.col[bb][l16][4 * g4]) : Tc[c];
          X = mfma16(Aop, Bop, X);
        }
        const bf16x4 Dop = *reinterpret_cast<const bf16x4*>(&sm.r2.d.row[a][l16][4 * g4]);
        const f32x4 Tv = mfma16(Dop, to_bf16x4(X), f32x4{0.f, 0.f, 0.f, 0.f});
        const float bc = sm.beta[16 * bb + l16];
        f32x4 Tn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Tn[j] = -Tv[j];
          sm.lb[16 * a + 4 * g4 + j][16 * bb + l16] = (bf16)(Tn[j] * bc);
        }
        Tc[a] = to_bf16x4(Tn);
      }
    }
    __syncthreads();

    // ---------------- Mq into the free A buffer; W = b X + L X with X = e^G k^ ----------------
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
      const int pi = wave + 4 * k3;
      if (pi >= 10) continue;
      int a, bb;
      pair_ab(pi, a, bb);
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.aoff[16 * a + 4 * g4 + j][16 * bb + l16] = (bf16)Mreg[k3][j];
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ct = wave + 4 * k2;  // 16-channel column tile of W
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const bf16x4 x4 = rows4(sm.ke, 16 * a + 4 * g4, 16 * ct, l16);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * a + 4 * g4]);
        f32x4 acc = bt * to_f32x4(x4);
#pragma unroll
        for (int ks = 0; ks < (a >= 2 ? 2 : 1); ++ks) {
          const bf16x8 Aop = *reinterpret_cast<const bf16x8*>(&sm.lb[16 * a + l16][32 * ks + 8 * g4]);
          const bf16x8 Bop = cat(rows4(sm.ke, 32 * ks + 8 * g4, 16 * ct, l16),
                                 rows4(sm.ke, 32 * ks + 8 * g4 + 4, 16 * ct, l16));
          acc = mfma32(Aop, Bop, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.r2.wn[16 * a + 4 * g4 + j][16 * ct + l16] = (bf16)(-acc[j]);
      }
    }
    __syncthreads();

    // ---------------- state-dependent part, per 16-column strip ----------------
    // (straight-line MFMA work; the next chunk's elementwise pass follows in the
    // same block so its VALU work can issue under these MFMAs)
    bf16x4 ob[SPW][4];
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const int s = wave + 4 * st;
      if constexpr (NS < 4) {
        if (s >= NS) break;
      }
      const int jl = 16 * s;
      bf16x8 Sb[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sb[kb] = cat(to_bf16x4(S[st][2 * kb]), to_bf16x4(S[st][2 * kb + 1]));

      // N = b V + L V - W S
      f32x4 N[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * rt + 4 * g4]);
        N[rt] = bt * to_f32x4(rows4(sm.v, 16 * rt + 4 * g4, jl, l16));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Bop = cat(rows4(sm.v, 32 * ks + 8 * g4, jl, l16),
                               rows4(sm.v, 32 * ks + 8 * g4 + 4, jl, l16));
#pragma unroll
        for (int rt = 2 * ks; rt < 4; ++rt) {
          const bf16x8 Aop = *reinterpret_cast<const bf16x8*>(&sm.lb[16 * rt + l16][32 * ks + 8 * g4]);
          N[rt] = mfma32(Aop, Bop, N[rt]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          N[rt] = mfma32(perm_row(sm.r2.wn, 16 * rt + l16, 32 * kb, g4), Sb[kb], N[rt]);

      // O = (e^G q) S + Mq N
      f32x4 O[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          O[rt] = mfma32(perm_row(sm.qe, 16 * rt + l16, 32 * kb, g4), Sb[kb], O[rt]);
      bf16x8 Nh[2], Nl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x4 h0 = to_bf16x4(N[2 * kb]), h1 = to_bf16x4(N[2 * kb + 1]);
        Nh[kb] = cat(h0, h1);
        Nl[kb] = cat(to_bf16x4(N[2 * kb] - to_f32x4(h0)), to_bf16x4(N[2 * kb + 1] - to_f32x4(h1)));
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rt = 2 * kb; rt < 4; ++rt)
          O[rt] = mfma32(perm_row(sm.aoff, 16 * rt + l16, 32 * kb, g4), Nh[kb], O[rt]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) ob[st][rt] = to_bf16x4(O[rt]);

      // S <- Diag(e^{G_last}) S + (e^{G_last - G} k)^T N, two-term split on both sides
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[16 * rt + 4 * g4]);
        S[st][rt] *= gm;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
          const bf16x8 Ah = cat(rows4(sm.kph, 32 * kb + 4 * g4, 16 * rt, l16),
                                rows4(sm.kph, 32 * kb + 16 + 4 * g4, 16 * rt, l16));
          const bf16x8 Al = cat(rows4(sm.kpl, 32 * kb + 4 * g4, 16 * rt, l16),
                                rows4(sm.kpl, 32 * kb + 16 + 4 * g4, 16 * rt, l16));
          S[st][rt] = mfma32(Ah, Nh[kb], S[st][rt]);
          S[st][rt] = mfma32(Ah, Nl[kb], S[st][rt]);
          S[st][rt] = mfma32(Al, Nh[kb], S[st][rt]);
        }
    }

    // elementwise pass of the next chunk (harmless recomputation after the last
    // one: nothing reads its results); it writes only rloc/wtot, which this
    // chunk no longer reads
    elementwise<VS>(el, pf, Ln, tq, g4, c2, c1, lb2, p.scale, &sm.rloc[wave][ch0],
                    &sm.wtot[wave][ch0]);

    // outputs (rows of tokens inside the sequence)
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const int s = wave + 4 * st;
      if constexpr (NS < 4) {
        if (s >= NS) break;
      }
      bf16* ocol = reinterpret_cast<bf16*>(outb) + 16 * s + l16;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (L == kC) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ocol[(unsigned)(t0 + 16 * rt + 4 * g4 + j) * ts_o] = ob[st][rt][j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = 16 * rt + 4 * g4 + j;
            if (t < L) ocol[(unsigned)(t0 + t) * ts_o] = ob[st][rt][j];
          }
        }
      }
    }
  }

  // final state
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    const int s = wave + 4 * st;
    if (s >= NS) break;
    const int jg = slice * VS + 16 * s + l16;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t idx = sbase + (size_t)(16 * rt + 4 * g4 + j) * kD + jg;
        if (p.state_bf16) static_cast<bf16*>(p.sT)[idx] = (bf16)S[st][rt][j];
        else static_cast<float*>(p.sT)[idx] = S[st][rt][j];
      }
  }
}

}  // namespace

hipError_t launch_chunk(const Params& p, hipStream_t stream) {
  const void* fn = nullptr;
  switch (kD / p.vsplit) {
    case 128: fn = reinterpret_cast<const void*>(&chunk_kernel<128>); break;
    case 64: fn = reinterpret_cast<const void*>(&chunk_kernel<64>); break;
    case 32: fn = reinterpret_cast<const void*>(&chunk_kernel<32>); break;
    case 16: fn = reinterpret_cast<const void*>(&chunk_kernel<16>); break;
    default: return hipErrorInvalidValue;
  }
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(p.N * p.H * p.vsplit), dim3(kThreads), args, 0, stream);
}

}  // namespace kda
