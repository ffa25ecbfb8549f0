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
// MFMA layout facts used here (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x16_bf16): lane l holds accumulator rows 4*(l/16)+j of
// column l%16.  Operand k-slots only have to agree between A and B, so a
// k-block of 32 built from two accumulator tiles uses the slot order
// {4g..4g+3, 16+4g..16+4g+3} (g = l/16) on both sides.
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kC = 64;  // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Blocks (a, b), b <= a, of the 4 x 4 block-lower-triangular chunk matrices.
__device__ __forceinline__ int blk(int a, int b) { return a * (a + 1) / 2 + b; }

template <int VS>
struct Smem {
  union {
    bf16 ke[kC][136];  // k^ e^{G-R}, rows = tokens (A left operand)
    struct {
      bf16 row[10][16][24];  // triangular-inverse blocks, row-major
      bf16 col[10][16][24];  // the same blocks transposed
    } tb;
    bf16 wn[kC][136];  // -W, rows = tokens
  } r0;
  bf16 qe[kC][136];     // (scale q^) e^{G-R}; later e^G (scale q^)
  bf16 kf[kC][136];     // k^ e^{R-G} (A/Mq right operand)
  bf16 xwt[128][72];    // e^G k^, [channel][token]
  bf16 kph[128][72];    // e^{G_last-G} k^, high bf16 part, [channel][token]
  bf16 kpl[128][72];    // low part
  float adiag[4][16][20];  // diagonal 16x16 blocks of A (fp32)
  bf16 aoff[kC][72];    // off-diagonal blocks of A; later Mq
  bf16 lb[kC][72];      // L = (Tm - I) diag(b), [token][token]
  bf16 vt[VS][72];      // V slice, [column][token]
  float beta[kC];
  float rloc[4][128];   // G at token 7 of each sub-chunk, relative to the sub-chunk
  float wtot[4][128];   // per-sub-chunk totals of the log-decay
  float dab[6][128];    // e^{R_a - R_b}, a > b
  float gam[128];       // e^{G_last}
};

// Global-memory values of one chunk, loaded one chunk ahead into registers.
// Thread (tq, co) = (tid / 16, tid % 16) covers tokens 4tq..4tq+3 and key
// channels 8co..8co+7 (q, k, g), and value columns co*VS/16 .. +VS/16-1.
template <int VS>
struct Prefetch {
  static constexpr int VN = VS / 16;  // value columns per thread
  uint4 q[4], k[4], g[4];
  bf16 v[4][VN];
  float beta;
};

template <int VS>
__device__ __forceinline__ void load_chunk(Prefetch<VS>& pf, const Params& p, int h, int slice,
                                           int t0, int L, int tq, int co, int tid) {
  const int H = p.H;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * tq + r;
    if (t < L) {
      const size_t base = ((size_t)(t0 + t) * H + h) * kD;
      pf.q[r] = *reinterpret_cast<const uint4*>(p.q + base + 8 * co);
      pf.k[r] = *reinterpret_cast<const uint4*>(p.k + base + 8 * co);
      pf.g[r] = *reinterpret_cast<const uint4*>(p.g + base + 8 * co);
      const bf16* vp = reinterpret_cast<const bf16*>(p.v + base + slice * VS + co * Prefetch<VS>::VN);
#pragma unroll
      for (int c = 0; c < Prefetch<VS>::VN; ++c) pf.v[r][c] = vp[c];
    } else {
      pf.q[r] = pf.k[r] = pf.g[r] = uint4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < Prefetch<VS>::VN; ++c) pf.v[r][c] = (bf16)0.f;
    }
  }
  pf.beta = (tid < L) ? bf16_to_f32(p.beta[(size_t)(t0 + tid) * H + h]) : 0.f;
}

__device__ __forceinline__ void unpack8(uint4 u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

__device__ __forceinline__ bf16x8 pack8(const float* f) {
  return bf16x8{(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3],
                (bf16)f[4], (bf16)f[5], (bf16)f[6], (bf16)f[7]};
}

// A-operand rows for a k-block of 32 whose B operand was built from two
// accumulator tiles: slots 0..3 <- columns base+4g.., slots 4..7 <- base+16+4g..
template <int STRIDE>
__device__ __forceinline__ bf16x8 perm_row(const bf16 (*arr)[STRIDE], int row, int base, int g4) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&arr[row][base + 4 * g4]);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&arr[row][base + 16 + 4 * g4]);
  return cat(lo, hi);
}

template <int VS>
__global__ __launch_bounds__(kThreads, 1) void chunk_kernel(Params p) {
  constexpr int NS = VS / 16;                 // 16-column strips in the slice
  constexpr int SPW = NS >= 4 ? NS / 4 : 1;   // strips per wave
  __shared__ __attribute__((aligned(16))) Smem<VS> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;  // MFMA lane coordinates
  const int tq = tid >> 4, co = tid & 15;     // elementwise coordinates
  const int ch0 = 8 * co;

  // workgroup -> (sequence rank, head, slice); consecutive work items (the
  // slices of one head) are kept on one XCD so they share q/k/g in its L2
  int b = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int slice = b % p.vsplit;
  const int rest = b / p.vsplit;
  const int h = rest % p.H;
  const int n = p.order[rest / p.H];
  const int H = p.H;

  // zero the triangular buffers whose upper blocks are never written
  for (int i = tid; i < kC * 72 / 8; i += kThreads) {
    reinterpret_cast<uint4*>(&sm.lb[0][0])[i] = uint4{0, 0, 0, 0};
    reinterpret_cast<uint4*>(&sm.aoff[0][0])[i] = uint4{0, 0, 0, 0};
  }

  // per-head constants: sigmoid argument in log2 units, lower bound in log2
  const float eA = expf(p.A_log[h]);
  const float c1 = -kLog2e * eA;
  float c2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c2[i] = c1 * p.dt_bias[h * kD + ch0 + i];
  const float lb2 = p.lower_bound * kLog2e;

  // state slice in accumulator layout: strip s, row tile rt, element j ->
  // S[16 rt + 4 g4 + j][16 s + l16] of this slice
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

  const int bos = min(max(p.cu[n], 0), p.T);
  const int eos = min(max(p.cu[n + 1], bos), p.T);

  Prefetch<VS> pf;
  if (bos < eos) load_chunk<VS>(pf, p, h, slice, bos, min(kC, eos - bos), tq, co, tid);

  for (int t0 = bos; t0 < eos; t0 += kC) {
    const int L = min(kC, eos - t0);
    __syncthreads();  // the previous chunk is done with every shared buffer

    // ---------------- elementwise: norms, gate, cumulative decay ----------------
    float qf[4][8], kf[4][8], lam[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unpack8(pf.q[r], qf[r]);
      unpack8(pf.k[r], kf[r]);
      unpack8(pf.g[r], lam[r]);
    }
    // value slice -> vt[column][token]; beta
#pragma unroll
    for (int c = 0; c < Prefetch<VS>::VN; ++c) {
      bf16x4 v4 = {pf.v[0][c], pf.v[1][c], pf.v[2][c], pf.v[3][c]};
      *reinterpret_cast<bf16x4*>(&sm.vt[co * Prefetch<VS>::VN + c][4 * tq]) = v4;
    }
    if (tid < kC) sm.beta[tid] = tid < L ? rcp(1.f + ex2(-kLog2e * pf.beta)) : 0.f;

    // the registers are free again: fetch the next chunk behind this one's compute
    if (t0 + kC < eos) load_chunk<VS>(pf, p, h, slice, t0 + kC, min(kC, eos - t0 - kC), tq, co, tid);

#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float qq = 0.f, kk = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qq = fmaf(qf[r][i], qf[r][i], qq);
        kk = fmaf(kf[r][i], kf[r][i], kk);
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        qq += __shfl_xor(qq, m, 16);
        kk += __shfl_xor(kk, m, 16);
      }
      const float rq = rsqrtf(qq + kNormEps) * p.scale;
      const float rk = rsqrtf(kk + kNormEps);
      const bool valid = 4 * tq + r < L;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qf[r][i] *= rq;
        kf[r][i] *= rk;
        // log2 of the decay: lb * sigmoid(exp(A_log) (g + dt_bias)) * log2(e)
        const float e = ex2(fmaf(lam[r][i], c1, c2[i]));
        lam[r][i] = valid ? lb2 * rcp(1.f + e) : 0.f;
      }
    }
    // inclusive cumulative sum over the chunk's tokens, per channel
#pragma unroll
    for (int r = 1; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) lam[r][i] += lam[r - 1][i];
    float rloc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tot = lam[3][i];
      float x = tot;
      float y = __shfl_up(x, 16, 64);
      if (g4 >= 1) x += y;
      y = __shfl_up(x, 32, 64);
      if (g4 >= 2) x += y;
      const float excl = x - tot;  // sum of earlier token groups of this sub-chunk
#pragma unroll
      for (int r = 0; r < 4; ++r) lam[r][i] += excl;  // now relative to the sub-chunk start
      rloc[i] = __shfl(lam[3][i], 16 + co, 64);       // token 7 of the sub-chunk
      if (g4 == 3) sm.wtot[wave][ch0 + i] = lam[3][i];
      if (g4 == 1) sm.rloc[wave][ch0 + i] = lam[3][i];
    }
    __syncthreads();

    // chunk-relative references and totals
    float R[8], GL[8], Rw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float pre = 0.f, all = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = sm.wtot[w][ch0 + i];
        if (w < wave) pre += wt;
        all += wt;
      }
      Rw[i] = pre;             // G just before this sub-chunk
      R[i] = pre + rloc[i];    // reference: G at token 7 of this sub-chunk
      GL[i] = all;             // G at the last token of the chunk
    }
    // per-channel tables shared by all waves
    for (int idx = tid; idx < 6 * 128; idx += kThreads) {
      const int pr = idx >> 7, c = idx & 127;
      const int a = pr < 1 ? 1 : pr < 3 ? 2 : 3;
      const int bb = pr - (a * (a - 1)) / 2;
      float d = sm.rloc[a][c] - sm.rloc[bb][c];
      for (int w = bb; w < a; ++w) d += sm.wtot[w][c];
      sm.dab[pr][c] = ex2(d);
    }
    if (tid < 16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.gam[ch0 + i] = ex2(GL[i]);
    }

    // operands
    float eR[8], eLR[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      eR[i] = ex2(R[i]);           // e^{R}, relative to the chunk start
      eLR[i] = ex2(GL[i] - R[i]);  // e^{G_last - R}
    }
    float xw[4][8], kph[4][8], kpl[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      float ke[8], qe[8], kfv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float Gt = lam[r][i] + Rw[i];  // chunk-relative G
        const float E = ex2(Gt - R[i]);
        const float F = ex2(R[i] - Gt);
        ke[i] = kf[r][i] * E;
        qe[i] = qf[r][i] * E;
        kfv[i] = kf[r][i] * F;
        const float kp = kfv[i] * eLR[i];  // e^{G_last - G_t} k^
        const float hi = (float)(bf16)kp;
        kph[r][i] = hi;
        kpl[r][i] = kp - hi;
      }
      const bf16x8 keb = pack8(ke);
      *reinterpret_cast<bf16x8*>(&sm.r0.ke[t][ch0]) = keb;
      *reinterpret_cast<bf16x8*>(&sm.qe[t][ch0]) = pack8(qe);
      *reinterpret_cast<bf16x8*>(&sm.kf[t][ch0]) = pack8(kfv);
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[r][i] = (float)keb[i] * eR[i];  // e^G k^ from the bf16 k^ e^{G-R}
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<bf16x4*>(&sm.xwt[ch0 + i][4 * tq]) =
          bf16x4{(bf16)xw[0][i], (bf16)xw[1][i], (bf16)xw[2][i], (bf16)xw[3][i]};
      *reinterpret_cast<bf16x4*>(&sm.kph[ch0 + i][4 * tq]) =
          bf16x4{(bf16)kph[0][i], (bf16)kph[1][i], (bf16)kph[2][i], (bf16)kph[3][i]};
      *reinterpret_cast<bf16x4*>(&sm.kpl[ch0 + i][4 * tq]) =
          bf16x4{(bf16)kpl[0][i], (bf16)kpl[1][i], (bf16)kpl[2][i], (bf16)kpl[3][i]};
    }
    __syncthreads();

    // ---------------- A and Mq blocks (bf16 MFMA over the 128 channels) ----------------
    f32x4 Mreg[3];
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
      const int pi = wave + 4 * k3;
      Mreg[k3] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pi >= 10) continue;
      const int a = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
      const int bb = pi - (a * (a + 1)) / 2;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c0 = 32 * ks + 8 * g4;
        const bf16x8 aK = *reinterpret_cast<const bf16x8*>(&sm.r0.ke[16 * a + l16][c0]);
        const bf16x8 aQ = *reinterpret_cast<const bf16x8*>(&sm.qe[16 * a + l16][c0]);
        bf16x8 bK = *reinterpret_cast<const bf16x8*>(&sm.kf[16 * bb + l16][c0]);
        if (bb < a) {
          const float* d = &sm.dab[(a * (a - 1)) / 2 + bb][c0];
          float f[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = (float)bK[i] * d[i];
          bK = pack8(f);
        }
        accA = mfma32(aK, bK, accA);
        accM = mfma32(aQ, bK, accM);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g4 + j;  // row inside the block
        const bool keepA = bb < a || l16 < r;
        const bool keepM = bb < a || l16 <= r;
        const float av = keepA ? accA[j] * sm.beta[16 * a + r] : 0.f;
        if (bb == a) sm.adiag[a][r][l16] = av;
        else sm.aoff[16 * a + r][16 * bb + l16] = (bf16)av;
        Mreg[k3][j] = keepM ? accM[j] : 0.f;
      }
    }
    __syncthreads();

    // ---------------- Tm = (I + A)^-1: diagonal blocks by forward substitution ----------------
    if (lane < 16) {
      const int a = wave, c = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc = fmaf(-sm.adiag[a][r][m], x[m], acc);
        x[r] = acc;
      }
      const int bi = blk(a, a);
      const float bc = sm.beta[16 * a + c];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.r0.tb.row[bi][r][c] = (bf16)x[r];
        sm.r0.tb.col[bi][c][r] = (bf16)x[r];
        sm.lb[16 * a + r][16 * a + c] = (bf16)((x[r] - (r == c ? 1.f : 0.f)) * bc);
      }
    }
    __syncthreads();

    // ---------------- off-diagonal blocks: T_ab = -D_a sum_c A_ac T_cb ----------------
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
      if (wave < 4 - lev) {
        const int a = wave + lev, bb = wave;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
        for (int c = bb; c < a; ++c) {
          const bf16x4 Aop = *reinterpret_cast<const bf16x4*>(&sm.aoff[16 * a + l16][16 * c + 4 * g4]);
          const bf16x4 Bop = *reinterpret_cast<const bf16x4*>(&sm.r0.tb.col[blk(c, bb)][l16][4 * g4]);
          X = mfma16(Aop, Bop, X);
        }
        const bf16x4 Dop = *reinterpret_cast<const bf16x4*>(&sm.r0.tb.row[blk(a, a)][l16][4 * g4]);
        f32x4 Tv = mfma16(Dop, to_bf16x4(X), f32x4{0.f, 0.f, 0.f, 0.f});
        const int bi = blk(a, bb);
        const float bc = sm.beta[16 * bb + l16];
        bf16x4 tcol;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float t = -Tv[j];
          tcol[j] = (bf16)t;
          sm.r0.tb.row[bi][4 * g4 + j][l16] = (bf16)t;
          sm.lb[16 * a + 4 * g4 + j][16 * bb + l16] = (bf16)(t * bc);
        }
        *reinterpret_cast<bf16x4*>(&sm.r0.tb.col[bi][l16][4 * g4]) = tcol;
      }
      __syncthreads();
    }

    // ---------------- Mq into the free A buffer; q operand -> e^G q; W ----------------
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
      const int pi = wave + 4 * k3;
      if (pi >= 10) continue;
      const int a = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
      const int bb = pi - (a * (a + 1)) / 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.aoff[16 * a + 4 * g4 + j][16 * bb + l16] = (bf16)Mreg[k3][j];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(&sm.qe[t][ch0]);
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (float)q8[i] * eR[i];
      *reinterpret_cast<bf16x8*>(&sm.qe[t][ch0]) = pack8(f);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ct = wave + 4 * k2;  // 16-channel column tile of W
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(&sm.xwt[16 * ct + l16][16 * a + 4 * g4]);
        f32x4 acc;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = sm.beta[16 * a + 4 * g4 + j] * (float)x4[j];
#pragma unroll
        for (int ks = 0; ks < (a >= 2 ? 2 : 1); ++ks) {
          const bf16x8 Aop = *reinterpret_cast<const bf16x8*>(&sm.lb[16 * a + l16][32 * ks + 8 * g4]);
          const bf16x8 Bop = *reinterpret_cast<const bf16x8*>(&sm.xwt[16 * ct + l16][32 * ks + 8 * g4]);
          acc = mfma32(Aop, Bop, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.r0.wn[16 * a + 4 * g4 + j][16 * ct + l16] = (bf16)(-acc[j]);
      }
    }
    __syncthreads();

    // ---------------- state-dependent part, per 16-column strip ----------------
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const int s = wave + 4 * st;
      if (s >= NS) break;
      const int jl = 16 * s + l16;
      const int jg = slice * VS + jl;
      bf16x8 Sb[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sb[kb] = cat(to_bf16x4(S[st][2 * kb]), to_bf16x4(S[st][2 * kb + 1]));

      // N = b V + L V - W S
      f32x4 N[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(&sm.vt[jl][16 * rt + 4 * g4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) N[rt][j] = sm.beta[16 * rt + 4 * g4 + j] * (float)v4[j];
#pragma unroll
        for (int ks = 0; ks < (rt >= 2 ? 2 : 1); ++ks) {
          const bf16x8 Aop = *reinterpret_cast<const bf16x8*>(&sm.lb[16 * rt + l16][32 * ks + 8 * g4]);
          const bf16x8 Bop = *reinterpret_cast<const bf16x8*>(&sm.vt[jl][32 * ks + 8 * g4]);
          N[rt] = mfma32(Aop, Bop, N[rt]);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) N[rt] = mfma32(perm_row(sm.r0.wn, 16 * rt + l16, 32 * kb, g4), Sb[kb], N[rt]);
      }

      // O = (e^G q) S + Mq N
      f32x4 O[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) O[rt] = mfma32(perm_row(sm.qe, 16 * rt + l16, 32 * kb, g4), Sb[kb], O[rt]);
      }
      bf16x8 Nh[2], Nl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x4 h0 = to_bf16x4(N[2 * kb]), h1 = to_bf16x4(N[2 * kb + 1]);
        Nh[kb] = cat(h0, h1);
        Nl[kb] = cat(to_bf16x4(N[2 * kb] - to_f32x4(h0)), to_bf16x4(N[2 * kb + 1] - to_f32x4(h1)));
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int kb = 0; kb < (rt >= 2 ? 2 : 1); ++kb)
          O[rt] = mfma32(perm_row(sm.aoff, 16 * rt + l16, 32 * kb, g4), Nh[kb], O[rt]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * rt + 4 * g4 + j;
          if (t < L) p.out[((size_t)(t0 + t) * H + h) * kD + jg] = f32_to_bf16(O[rt][j]);
        }
      }

      // S <- Diag(e^{G_last}) S + (e^{G_last - G} k)^T N, two-term split on both sides
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[16 * rt + 4 * g4]);
        S[st][rt] *= gm;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 Ah = perm_row(sm.kph, 16 * rt + l16, 32 * kb, g4);
          const bf16x8 Al = perm_row(sm.kpl, 16 * rt + l16, 32 * kb, g4);
          S[st][rt] = mfma32(Ah, Nh[kb], S[st][rt]);
          S[st][rt] = mfma32(Ah, Nl[kb], S[st][rt]);
          S[st][rt] = mfma32(Al, Nh[kb], S[st][rt]);
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
        if (p.state_bf16) static_cast<uint16_t*>(p.sT)[idx] = f32_to_bf16(S[st][rt][j]);
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
