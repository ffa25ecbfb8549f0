// kda_fwd32.hip -- KDA chunked-prefill forward for gfx950 on 32-token chunks.
//
// The method is the bounded-gate, normalised-q/k delta rule of vLLM PR
// #55737's report ("Features and motivation"):
//   S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale S_t^T q_t,
// with log a_t = lower_bound * sigmoid(exp(A_log) (g_t + dt_bias)), b_t =
// sigmoid(beta logit) and q, k L2-normalised.  Over a chunk, with G the
// inclusive cumulative log-decay per key channel and S the state entering it:
//   A[t,i] = b_t sum_c k_t[c] k_i[c] e^{G_t[c]-G_i[c]}        (i < t)
//   M[t,i] = scale sum_c q_t[c] k_i[c] e^{G_t[c]-G_i[c]} / |q_t|   (i <= t)
//   N = (I + A)^-1 diag(b) (V - (e^G k) S)
//   O = scale (e^G q) S / |q| + M N
//   S <- Diag(e^{G_last}) S + (e^{G_last - G} k)^T N
//
// Halves and exponent ranges.  A chunk is two 16-token halves h, each with its
// own reference point (the start of the half): G^h is the cumulative decay
// from the half's start, Gam_h = e^{G^h_last} the half's total decay.  Per
// half, with k~ = k / |k|:
//   X^h = e^{G^h} k~,  Q^h = e^{G^h} q,  K'^h = e^{G^h_last - G^h} k~,
//   K_G^h = e^{-G^h} k~ = K'^h / Gam_h
// X^h, K'^h <= 1 and |Q^h| <= |q|, while K_G^h grows up to
// 2^{16 |lower_bound| log2 e} <= 2^127 for lower_bound >= -5.5.  The chunk's
// terms in these operands:
//   A_hh = diag(b) X^h K_G^hT (diagonal blocks), A_10 = diag(b) X^1 K'^0T
//   (second half against the first: e^{G_t - G_i} = e^{G^1_t} e^{G^0_last - G^0_i}),
//   M likewise with Q^h, and the state enters through
//   Y_0 = X^0 S, Y_1 = X^1 (Gam_0 S)      (e^{G_t} for t in the second half is Gam_0 e^{G^1_t})
//   S_mid = Gam_0 S + K'^0T N_0           (the state after the first half)
//   S <- Gam_1 S_mid + K'^1T N_1.
// Pairs t < i (masked) may overflow; they are dropped by selects.
//
// Work split.  One workgroup per (sequence, head, value slice).  Four
// "producer" waves, two per chunk slot (one per half), build the packages of
// alternating chunks: norms, gate, cumulative decay and the decayed operands
// of their half (16 tokens x 128 channels), then, once both halves are in
// LDS, one forms A and the inverse (I + A)^-1, the other M.  None of it
// depends on the state.  The "state waves" (one or two 16-column strips of the
// value slice each) walk the chunks in order with their strips of S (128 x 16
// fp32) in registers.  No workgroup barrier in the main loops: LDS counters
// say which halves formed their operands, which finished their products, and
// which chunks each state wave is done with; packages are double-buffered per
// slot.
//
// Precision (checked against the fp64 recurrence on the workloads'
// distributions by an emulation of every rounding step): bf16 MFMA operands
// with fp32 accumulation; the 16x16 inverses by MFMA doubling, the
// off-diagonal block by two products; the state update in fp16 operands
// (K' / 16 and N / 16, both scalings exact).
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kC = 32;      // tokens per chunk
constexpr int kHT = 16;     // tokens per half
constexpr int kSlots = 2;   // chunk slots (producer wave pairs)
constexpr int kProd = 2 * kSlots;
constexpr int kSpinMax = 1 << 22;  // polls before a wait gives up (then the error word is set)
// Exponent shift of the decayed operands: X and Q carry 2^8, K_G 2^-8 and
// the fp16 K' 2^-4, and the state waves hold 2^-8 S.  With lower_bound
// >= -5.5 a half's decay spans 2^{+-126.96}; shifted, every operand factor
// lies in [2^-119, 2^119], so none is a denormal (which the hardware flushes:
// e^{G_t} of a half's last token and its K_G partner meet in M's diagonal).
constexpr float kShift = 8.f;
constexpr float kSDown = 1.f / 256.f;  // state held as 2^-8 S
constexpr float kSUp = 256.f;

template <int VS>
struct Cfg32 {
  static constexpr int NS = VS / 16;             // 16-column strips in the slice
  static constexpr int NSW = NS < 4 ? NS : 4;    // state waves
  static constexpr int SPW = NS / NSW;           // strips per state wave
  static constexpr int kThreads = 64 * (kProd + NSW);
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ---- LDS layouts ---------------------------------------------------------------
// Token-row operands ([32 tokens][128 channels] bf16): the 16-byte unit u of
// row t sits at unit u ^ (t & 15), so that both the producers' row writes (16
// lanes: one row, 16 units) and the MFMA operand reads (16 lanes: 16 rows, one
// unit) touch distinct banks.
__device__ __forceinline__ int tro(int t, int u) { return t * 128 + ((u ^ (t & 15)) << 3); }

// K' / 16 (fp16) as [32 tokens][128 keys in state-row order].  The state
// strip's accumulator tile rt holds, in lane group g4 register j, key
// pi(16 rt + 4 g4 + j) = 32 (rt >> 1) + 8 g4 + 4 (rt & 1) + j: then a lane's
// eight keys of a 32-key block are consecutive, which is what the Y = X S
// product needs from S as its B operand.  The update's A operand K'^T must
// follow the same row order.  8-byte unit U = 8 kb + 4 hi + g (keys
// pi(16 (2 kb + hi) + 4 g .. + 3)) sits at (16 hi + 4 kb + g) ^ (4 (t & 3)).
__device__ __forceinline__ int kpo(int t, int kb, int hi, int g) {
  return t * 128 + ((((hi << 4) | (kb << 2) | g) ^ ((t & 3) << 2)) << 2);
}

// Gamma vectors in the state waves' read order: key 32 kb + 8 g4 + 2 p + e at
// 32 g4 + 8 kb + 2 p + e, so lane 16 g4 + 4 kb + p reads its two keys as one
// 8-byte word and a wave reads the 512 bytes in order.
__device__ __forceinline__ int gmo(int key) {
  return ((key >> 3) & 3) * 32 + (key >> 5) * 8 + (key & 7);
}

struct Pack {
  bf16 x[kC * 128];        // 2^8 X^h, token rows (tro)
  bf16 qt[kC * 128];       // 2^8 Q^h, token rows (tro)
  _Float16 kp[kC * 128];   // K'^h / 16, token rows in state-row key order (kpo)
  bf16 l[2][512];          // L / 16 = ((I + A)^-1 - I) diag(b) / 16, A fragments of row block p
  bf16 m[2][512];          // 16 M', A fragments of row block p
  float gam[2][128];       // Gam_0, Gam_1 (gmo order)
  float b16[kC];           // b / 16
  float rqs[kC];           // scale / |q|
};

struct Scratch {           // per slot, read only by the products of the same chunk
  bf16 kg[kC * 128];       // 2^-8 K_G^h, token rows (tro)
  bf16 kp0[kHT * 128];     // bf16(K'^0 / 16), token rows (tro)
};

// Per state wave and strip: V rows -> accumulator layout, O accumulator ->
// rows (two 16-token blocks, 512 bytes each; the V reads of a block complete
// before its O writes).
struct Tile {
  bf16 t[2][256];
};

// LDS counters, all counted over the run (so a count names a chunk).
struct Sync {
  int done[kSlots][4];   // per state wave: chunks of this slot it is done with
  int opnd[kSlots];      // per producer slot: halves whose operands are in LDS (two per chunk)
  int rdy[kSlots][2];    // per package buffer: four per complete package (products: 2 + 2)
  int err;               // a bounded wait gave up (its kind)
  int pad;
};

template <int NSW, int SPW>
struct Smem {
  Pack pk[kSlots][2];
  Scratch sc[kSlots];
  Tile tl[NSW][SPW];
  Sync sy;
};

// ---- waits -------------------------------------------------------------------
__device__ __forceinline__ void arrive(int* ctr, int lane) {
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until *ctr >= target.  Every count is produced by waves that do not
// wait, directly or through others, for the waiting wave, so the wait ends;
// the bound keeps a broken count from holding the device, and giving up is
// recorded (err) so the call can report it.
__device__ __forceinline__ bool gave_up(const int* err) {
  // an LDS word: an atomic load keeps it a ds_read (a volatile generic read
  // becomes a flat load, whose wait also drains every vector memory operation)
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
}
// Record a give-up: the first one's kind stays (status word values).
constexpr int kErrWait = 1;  // a wait on this workgroup's LDS counters
__device__ __forceinline__ void give_up(int* err, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_count(const int* ctr, int target, int* err) {
  if (gave_up(err)) return;  // an earlier wait gave up: the results are void, finish quickly
#pragma unroll 1
  for (int it = 0; it < kSpinMax; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  give_up(err, kErrWait);
}

// Wait until the first n counters of a 16-byte row are all >= target (one
// LDS read per poll).
template <int n>
__device__ __forceinline__ void wait_row(const int* row, int target, int* err) {
  if (gave_up(err)) return;
#pragma unroll 1
  for (int it = 0; it < kSpinMax; ++it) {
    typedef __attribute__((address_space(3))) const volatile i32x4 lds_row;
    const i32x4 d = *(lds_row*)(row);
    int m = d[0];
    if (n > 1) m = min(m, d[1]);
    if (n > 2) m = min(m, min(d[2], d[3]));
    if (__builtin_amdgcn_readfirstlane(m) >= target) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  give_up(err, kErrWait);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Add n to an LDS counter (release).
__device__ __forceinline__ void arrive_n(int* ctr, int lane, int n) {
  if (lane == 0) __hip_atomic_fetch_add(ctr, n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---- small helpers --------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;
// Buffer resource over one head's rows, bounded at the sequence end (loads past
// it return 0, stores past it are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int eos, int rowstride,
                                                          int rowlen) {
  const unsigned bytes = eos > 0 ? (unsigned(eos - 1) * unsigned(rowstride) + unsigned(rowlen)) * 2u : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcWord3);
}

// (bound_ctrl set: every lane is written, so the move can fold into its user)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of a row, result in every lane of the row
__device__ __forceinline__ float row_sum(float s) {
  s += dpp<0x128>(s);  // row_ror:8
  s += dpp<0x124>(s);  // row_ror:4
  s += dpp<0x4E>(s);   // quad_perm [2,3,0,1]
  s += dpp<0xB1>(s);   // quad_perm [1,0,3,2]
  return s;
}
// lane N of this lane's row of 16 (row_newbcast)
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, true));
}

__device__ __forceinline__ float dot2(uint32_t a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, a), c,
                                         false);
}
__device__ __forceinline__ uint32_t pkb(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}
__device__ __forceinline__ uint32_t pkh(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
}
__device__ __forceinline__ float chan8(const uint4& w, int s) {
  const uint32_t d = s < 2 ? w.x : s < 4 ? w.y : s < 6 ? w.z : w.w;
  return (s & 1) ? bf16_hi(d) : bf16_lo(d);
}
__device__ __forceinline__ bf16x8 lds16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f16x4 tr4h(const _Float16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}
__device__ __forceinline__ f32x4 mfma16x(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// ---- producer: raw loads ----------------------------------------------------------
// One half of a chunk (16 tokens, all 128 channels) per producer wave: lane
// (tq = lane / 16, cg = lane % 16) holds tokens 4 tq + i (i = 0..3) of the
// half, channels 8 cg .. + 7 (one 16-byte unit), so 16 consecutive lanes read
// one 256-byte row.  The per-chunk part of each byte offset is a scalar
// (soffset); the lane part is fixed.
struct Raw {
  uint4 q[4], k[4], g[4];
  uint32_t beta;
};

struct Loader {
  __amdgpu_buffer_rsrc_t q, k, g, beta;
  unsigned vq, vk, vg, vb;  // lane parts of the byte offsets
  int ts_q, ts_k, ts_g, ts_b;
  __device__ __forceinline__ void init(int lane) {
    const unsigned tq = unsigned(lane >> 4), cg = unsigned(lane & 15);
    vq = (4u * tq * unsigned(ts_q) + 8u * cg) * 2u;
    vk = (4u * tq * unsigned(ts_k) + 8u * cg) * 2u;
    vg = (4u * tq * unsigned(ts_g) + 8u * cg) * 2u;
    vb = cg * unsigned(ts_b) * 2u;
  }
  __device__ __forceinline__ void gate(Raw& r, int t0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.g[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g, vg, (unsigned(t0) + i) * unsigned(ts_g) * 2u, 0));
    r.beta = __builtin_amdgcn_raw_buffer_load_b16(beta, vb, unsigned(t0) * unsigned(ts_b) * 2u, 0);
  }
  __device__ __forceinline__ void qk(Raw& r, int t0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k, vk, (unsigned(t0) + i) * unsigned(ts_k) * 2u, 0));
      r.q[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(q, vq, (unsigned(t0) + i) * unsigned(ts_q) * 2u, 0));
    }
  }
};

// ---- producer: operands of one half --------------------------------------------------
// Writes 2^8 X, 2^8 Q, K' / 16 (package), 2^-8 K_G and (first half) bf16(K'^0
// / 16) (scratch) of the half, Gam_h, b / 16 and scale / |q| of its tokens.
// nvalid: tokens of the half inside the sequence (0..16).  The next loads
// (token tn) are issued as soon as their registers are consumed.
template <int HF>
__device__ __forceinline__ void produce_half(Pack& P, Scratch& SC, Raw& raw, const Loader& ld, int tn,
                                             int nvalid, int lane, const float (&c2)[8], float c1,
                                             float lb2, float scale) {
  const int cg = lane & 15, tq = lane >> 4;
  // norms of the lane's 4 tokens (8 channels per lane, 16 lanes per row)
  float rk[4], rq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 kk = raw.k[i], qq = raw.q[i];
    rk[i] = __builtin_amdgcn_rsqf(row_sum(dot2(kk.w, dot2(kk.z, dot2(kk.y, dot2(kk.x, 0.f))))) + kNormEps);
    rq[i] = __builtin_amdgcn_rsqf(row_sum(dot2(qq.w, dot2(qq.z, dot2(qq.y, dot2(qq.x, 0.f))))) + kNormEps) * scale;
  }
  // gate sigma per (token, channel) and its running sum over the lane's 4
  // tokens; tokens past the sequence end get 1 / inf = 0
  float cs[8][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pad = 4 * tq + i < nvalid ? 1.f : __builtin_inff();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float sg = rcp(ex2(fmaf(chan8(raw.g[i], s), c1, c2[s])) + pad);
      cs[s][i] = i == 0 ? sg : cs[s][i - 1] + sg;
    }
  }
  // beta / 16 of token cg of the half (lanes < 16), zero past the end
  const float bet = cg < nvalid ? rcp(1.f + ex2(-kLog2e * bf16_to_f32(uint16_t(raw.beta)))) * 0.0625f : 0.f;
  __builtin_amdgcn_sched_barrier(0);
  ld.gate(raw, tn);  // next gate inputs and beta logit
  __builtin_amdgcn_sched_barrier(0);
  if (tq == 0) P.b16[kHT * HF + cg] = bet;
  if (cg == 0) *reinterpret_cast<f32x4*>(&P.rqs[kHT * HF + 4 * tq]) = f32x4{rq[0], rq[1], rq[2], rq[3]};
  // earlier token groups' sums (rows of 16 lanes) and the half's total, per channel
  float ex[8], tot[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const unsigned t = __float_as_uint(cs[s][3]);
    const auto pr = __builtin_amdgcn_permlane16_swap(t, t, false, false);
    const float te = __uint_as_float(pr[0]), to = __uint_as_float(pr[1]);  // rows tq & ~1, tq | 1
    const unsigned pp = __float_as_uint(te + to);
    const auto pq2 = __builtin_amdgcn_permlane32_swap(pp, pp, false, false);
    const float p01 = __uint_as_float(pq2[0]), p23 = __uint_as_float(pq2[1]);
    ex[s] = ((tq & 2) ? p01 : 0.f) + ((tq & 1) ? te : 0.f);
    tot[s] = p01 + p23;
  }
  float ginv16[8];  // Gam_h^-1 / 16
#pragma unroll
  for (int s = 0; s < 8; ++s) ginv16[s] = ex2(-lb2 * tot[s] - 4.f);
  if (tq == 0) {
    float gam[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) gam[s] = ex2(lb2 * tot[s]);
    *reinterpret_cast<f32x4*>(&P.gam[HF][gmo(8 * cg)]) = f32x4{gam[0], gam[1], gam[2], gam[3]};
    *reinterpret_cast<f32x4*>(&P.gam[HF][gmo(8 * cg) + 4]) = f32x4{gam[4], gam[5], gam[6], gam[7]};
  }
  const int kb = cg >> 2, g = cg & 3;  // K' units (kpo): keys 8 cg + 4 hi .. + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = kHT * HF + 4 * tq + i;
    float vx[8], vq[8], vk[8], vg[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float el = lb2 * ex[s];
      const float E = ex2(fmaf(cs[s][i], lb2, el + kShift));                   // 2^8 e^{G}
      const float Kq = ex2(fmaf(cs[s][i], -lb2, lb2 * tot[s] - el - 4.f));    // e^{G_last - G} / 16
      const float kt = chan8(raw.k[i], s) * rk[i];
      vx[s] = E * kt;
      vq[s] = E * chan8(raw.q[i], s);
      vk[s] = Kq * kt;                                        // K' / 16
      vg[s] = vk[s] * ginv16[s];                              // 2^-8 K_G
    }
    const int o = tro(t, cg);
    *reinterpret_cast<uint4*>(&P.x[o]) = uint4{pkb(vx[0], vx[1]), pkb(vx[2], vx[3]), pkb(vx[4], vx[5]), pkb(vx[6], vx[7])};
    *reinterpret_cast<uint4*>(&P.qt[o]) = uint4{pkb(vq[0], vq[1]), pkb(vq[2], vq[3]), pkb(vq[4], vq[5]), pkb(vq[6], vq[7])};
    *reinterpret_cast<uint4*>(&SC.kg[o]) = uint4{pkb(vg[0], vg[1]), pkb(vg[2], vg[3]), pkb(vg[4], vg[5]), pkb(vg[6], vg[7])};
    *reinterpret_cast<uint2*>(&P.kp[kpo(t, kb, 0, g)]) = uint2{pkh(vk[0], vk[1]), pkh(vk[2], vk[3])};
    *reinterpret_cast<uint2*>(&P.kp[kpo(t, kb, 1, g)]) = uint2{pkh(vk[4], vk[5]), pkh(vk[6], vk[7])};
    if constexpr (HF == 0)
      *reinterpret_cast<uint4*>(&SC.kp0[o]) = uint4{pkb(vk[0], vk[1]), pkb(vk[2], vk[3]), pkb(vk[4], vk[5]), pkb(vk[6], vk[7])};
  }
  __builtin_amdgcn_sched_barrier(0);
  ld.qk(raw, tn);  // next q and k
}

// ---- producer: products ---------------------------------------------------------------
// A-operand fragments (16 tokens from row t0, k = 128 channels in 4 blocks of
// 32) of a token-row tile: lane (l16, g4) holds row t0 + l16, channels
// 32 kb + 8 g4 .. + 7.
__device__ __forceinline__ void rows_frag(const bf16* base, int t0, int lane, bf16x8 (&f)[4]) {
  const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) f[kb] = lds16(base + tro(t0 + l16, 4 * kb + g4));
}

// (I + A)^-1 of a strictly lower 16x16 A given accumulator(A) (lane (l16, g4)
// register j: A[4 g4 + j][l16]) and accumulator(A^T): the doubling
// (I - A)(I + A^2)(I + A^4)(I + A^8), each product formed together with its
// transpose.  An accumulator(Z) register set is Z's B operand and Z^T's A
// operand.  Returns accumulator(T^T), T = (I + A)^-1.
__device__ __forceinline__ f32x4 inv16(f32x4 Nn, f32x4 Nt, f32x4 I4) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const bf16x4 nb = to_bf16x4(Nn), ntb = to_bf16x4(Nt);
  const f32x4 N2 = mfma16(ntb, nb, zero), N2t = mfma16(nb, ntb, zero);
  const bf16x4 n2b = to_bf16x4(N2), n2tb = to_bf16x4(N2t);
  const f32x4 N4 = mfma16(n2tb, n2b, zero), N4t = mfma16(n2b, n2tb, zero);
  const bf16x4 n4b = to_bf16x4(N4), n4tb = to_bf16x4(N4t);
  const f32x4 N8 = mfma16(n4tb, n4b, zero);
  const f32x4 P1t = mfma16(n2b, to_bf16x4(-Nt), I4 - Nt + N2t);  // (I - A)(I + A^2)
  const f32x4 P2t = mfma16(n4b, to_bf16x4(P1t), P1t);              // ... (I + A^4)
  return mfma16(to_bf16x4(N8), to_bf16x4(P2t), P2t);               // ... (I + A^8)
}

// First-half wave: A, (I + A)^-1 and L / 16 for the state's N product.
__device__ __forceinline__ void produce_inverse(Pack& P, const Scratch& SC, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  bf16x8 xa[4], ka[4];
  // diagonal block h: A_hh = diag(b) X^h K_G^hT, masked to i < t
  f32x4 Nn[2], Nt[2];
  const f32x4 b4[2] = {*reinterpret_cast<const f32x4*>(&P.b16[4 * g4]),
                       *reinterpret_cast<const f32x4*>(&P.b16[kHT + 4 * g4])};
  const float bc[2] = {P.b16[l16], P.b16[kHT + l16]};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    rows_frag(P.x, kHT * h, lane, xa);
    rows_frag(SC.kg, kHT * h, lane, ka);
    f32x4 a = zero, at = zero;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      a = mfma32(xa[kb], ka[kb], a);    // [t = 4 g4 + j][i = l16]
      at = mfma32(ka[kb], xa[kb], at);  // [i = 4 g4 + j][t = l16] = A[l16][4 g4 + j]
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g4 + j;
      Nn[h][j] = l16 < r ? 16.f * b4[h][j] * a[j] : 0.f;    // A[r][l16]
      Nt[h][j] = r < l16 ? 16.f * bc[h] * at[j] : 0.f;      // A[l16][r]
    }
  }
  // off-diagonal block A_10 = diag(b_1) X^1 K'^0T (2^8 X^1 against K'^0 / 16, b16 = b / 16)
  bf16x8 ka0[4];
  rows_frag(P.x, kHT, lane, xa);
  rows_frag(SC.kp0, 0, lane, ka0);
  f32x4 a10 = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) a10 = mfma32(xa[kb], ka0[kb], a10);  // [t = 16 + 4 g4 + j][i = l16]
  a10 = a10 * b4[1];
  f32x4 I4;
#pragma unroll
  for (int j = 0; j < 4; ++j) I4[j] = 4 * g4 + j == l16 ? 1.f : 0.f;
  const f32x4 Dt0 = inv16(Nn[0], Nt[0], I4);  // accumulator(T_00^T): T_00[l16][4 g4 + j]
  const f32x4 Dt1 = inv16(Nn[1], Nt[1], I4);
  // T_10 = -T_11 A_10 T_00 as accumulator(T_10^T) = -T_00^T (A_10^T T_11^T)
  const f32x4 D0 = mfma16(to_bf16x4(Dt0), to_bf16x4(I4), zero);          // accumulator(T_00)
  const f32x4 W = mfma16(to_bf16x4(a10), to_bf16x4(Dt1), zero);          // accumulator(A_10^T T_11^T)
  const f32x4 T10t = -mfma16(to_bf16x4(D0), to_bf16x4(W), zero);         // T_10[l16][4 g4 + j]
  // L / 16 = (T - I) diag(b) / 16, row block p: lane (l16 = t, g4) holds
  // columns 4 g4 + j (first half) and 16 + 4 g4 + j (second half)
  const f32x4 l00 = (Dt0 - I4) * b4[0];
  const f32x4 l10 = T10t * b4[0];
  const f32x4 l11 = (Dt1 - I4) * b4[1];
  *reinterpret_cast<bf16x8*>(&P.l[0][8 * lane]) = cat(to_bf16x4(l00), to_bf16x4(zero));
  *reinterpret_cast<bf16x8*>(&P.l[1][8 * lane]) = cat(to_bf16x4(l10), to_bf16x4(l11));
}

// Second-half wave: 16 M' = 16 rqs (Q K_G^T) (diagonal blocks, i <= t) and
// 16 rqs Q^1 K'^0T (off-diagonal), as A fragments of the state's O product.
__device__ __forceinline__ void produce_m(Pack& P, const Scratch& SC, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  bf16x8 qa[4], ka[4];
  f32x4 mt[3];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    rows_frag(P.qt, kHT * h, lane, qa);
    rows_frag(SC.kg, kHT * h, lane, ka);
    f32x4 a = zero;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) a = mfma32(ka[kb], qa[kb], a);  // [i = 4 g4 + j][t = l16]
    const float r16 = 16.f * P.rqs[kHT * h + l16];
#pragma unroll
    for (int j = 0; j < 4; ++j) mt[h][j] = 4 * g4 + j <= l16 ? r16 * a[j] : 0.f;
  }
  rows_frag(SC.kp0, 0, lane, ka);  // qa still holds Q^1
  f32x4 a = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) a = mfma32(ka[kb], qa[kb], a);
  mt[2] = a * P.rqs[kHT + l16];  // 2^8 Q^1 against K'^0 / 16: 16 M'
  *reinterpret_cast<bf16x8*>(&P.m[0][8 * lane]) = cat(to_bf16x4(mt[0]), to_bf16x4(zero));
  *reinterpret_cast<bf16x8*>(&P.m[1][8 * lane]) = cat(to_bf16x4(mt[2]), to_bf16x4(mt[1]));
}

// S <- Diag(Gam) S on one strip: each lane read two factors (gmo order), the
// rest arrive by row broadcast: register (rt, j) is key
// pi(16 rt + 4 g4 + j), factor in lane 2 rt + j / 2 of the row, component j % 2.
template <int RT = 0>
__device__ __forceinline__ void decay_strip(f32x4 (&S)[8], float g0, float g1) {
  S[RT][0] = S[RT][0] * row_bcast<2 * RT>(g0);
  S[RT][1] = S[RT][1] * row_bcast<2 * RT>(g1);
  S[RT][2] = S[RT][2] * row_bcast<2 * RT + 1>(g0);
  S[RT][3] = S[RT][3] * row_bcast<2 * RT + 1>(g1);
  if constexpr (RT < 7) decay_strip<RT + 1>(S, g0, g1);
}

__device__ __forceinline__ uint2 load_vrow(__amdgpu_buffer_rsrc_t v, unsigned c0, int rowstride, int t0,
                                           int lane) {
  const unsigned off =
      ((unsigned(t0) + unsigned(lane >> 2)) * unsigned(rowstride) + c0 + 4u * unsigned(lane & 3)) * 2u;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(v, off, 0, 0));
}

template <int VS, bool CK>
__global__ __launch_bounds__(Cfg32<VS>::kThreads, 1) void fwd32_kernel(Params p) {
  using C = Cfg32<VS>;
  constexpr int SPW = C::SPW, NSW = C::NSW;
  __shared__ __attribute__((aligned(16))) Smem<NSW, SPW> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int b = work_item(blockIdx.x, gridDim.x, p.vsplit);
  const int slice = b % p.vsplit;
  const int rest = b / p.vsplit;
  const int h = rest % p.H;
  const int H = p.H;
  if (tid < int(sizeof(Sync) / sizeof(int))) reinterpret_cast<int*>(&sm.sy)[tid] = 0;
  int n;
  if (p.order) {
    n = p.order[rest / H];
  } else {
    int* seq_sh = reinterpret_cast<int*>(sm.pk[1][1].gam);
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
    n = __builtin_amdgcn_readfirstlane(seq_sh[0]);
  }
  __syncthreads();

  // the bounds are uniform: scalar registers (else every buffer access with a
  // token offset in its scalar operand becomes a loop over lanes)
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n + 1], bos), p.T));
  const int nc = (eos - bos + kC - 1) / kC;   // chunks
  int* err = &sm.sy.err;

  // ---------------- producer waves: wave = 2 slot + half ----------------
  // Two producer slots of two waves each: slot k builds chunks k, k + 2, ..,
  // wave (k, HF) the operands of half HF; then one of the two forms A and the
  // inverse, the other M (alternating between chunks).
  auto producer = [&](auto kq, auto hq) {
    constexpr int K = decltype(kq)::value, HF = decltype(hq)::value;
    Loader ld;
    ld.q = rows_rsrc(p.q + size_t(h) * p.hs_q, eos, p.ts_q, kD);
    ld.k = rows_rsrc(p.k + size_t(h) * p.hs_k, eos, p.ts_k, kD);
    ld.g = rows_rsrc(p.g + size_t(h) * p.hs_g, eos, p.ts_g, kD);
    ld.beta = rows_rsrc(p.beta + size_t(h) * p.hs_b, eos, p.ts_b, 1);
    ld.ts_q = p.ts_q, ld.ts_k = p.ts_k, ld.ts_g = p.ts_g, ld.ts_b = p.ts_b;
    ld.init(lane);
    const float eA = expf(p.A_log[h]);
    const float c1 = -kLog2e * eA;
    const float lb2 = p.lower_bound * kLog2e;
    float c2[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) c2[s] = c1 * p.dt_bias[h * kD + 8 * (lane & 15) + s];
    __builtin_amdgcn_sched_barrier(0);
    Raw raw;
    ld.gate(raw, bos + kC * K + kHT * HF);
    ld.qk(raw, bos + kC * K + kHT * HF);
#pragma unroll 1
    for (int j = K; j < nc; j += 2) {
      const int u = j >> 1, bf = u & 1;  // the slot's u-th chunk, package buffer bf
      Pack& P = sm.pk[K][bf];
      Scratch& SC = sm.sc[K];
      // the package buffer is free once every state wave is done with chunk
      // j - 4, the scratch once the products of chunk j - 2 are
      if (j >= 4) wait_row<NSW>(sm.sy.done[K], u - 1, err);
      if (j >= 2) wait_count(&sm.sy.rdy[K][bf ^ 1], 4 * (((u - 1) >> 1) + 1), err);
      const int t0 = bos + kC * j + kHT * HF;
      produce_half<HF>(P, SC, raw, ld, t0 + 2 * kC, min(kHT, max(eos - t0, 0)), lane, c2, c1, lb2, p.scale);
      arrive(&sm.sy.opnd[K], lane);
      wait_count(&sm.sy.opnd[K], 2 * (u + 1), err);
      if (HF == (u & 1)) produce_inverse(P, SC, lane);
      else produce_m(P, SC, lane);
      arrive_n(&sm.sy.rdy[K][bf], lane, 2);
    }
  };
  if (wave < kProd) {
    switch (wave) {
      case 0: producer(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}); break;
      case 1: producer(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}); break;
      case 2: producer(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}); break;
      default: producer(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); break;
    }
    if (lane == 0 && gave_up(err)) p.errword[0] = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return;
  }

  // ---------------- state waves ----------------
  __builtin_amdgcn_s_setprio(2);
  const int sw = wave - kProd;
  const int colb = slice * VS + 16 * sw + l16;  // column of strip 0 (strip u adds 16 NSW u)
  const __amdgpu_buffer_rsrc_t vsrc = rows_rsrc(p.v + size_t(h) * p.hs_v, eos, p.ts_v, kD);
  const __amdgpu_buffer_rsrc_t odst = rows_rsrc(p.out + size_t(h) * p.hs_o, eos, p.ts_o, kD);
  const size_t sbase = (size_t(n) * H + h) * kD * kD;
  // S[u][rt][j] = 2^-8 S[key pi(16 rt + 4 g4 + j)][column of strip u]
  f32x4 S[SPW][8];
  auto key_of = [&](int rt, int j) { return 32 * (rt >> 1) + 8 * g4 + 4 * (rt & 1) + j; };
  // strip u of S, in the state dtype, into the [D, D] block at dst + base
  auto store_strip = [&](void* dst, size_t base, int u) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const size_t o = base + size_t(key_of(rt, jj)) * kD + colb + 16 * NSW * u;
        if (p.state_bf16) static_cast<bf16*>(dst)[o] = (bf16)(S[u][rt][jj] * kSUp);
        else static_cast<float*>(dst)[o] = S[u][rt][jj] * kSUp;
      }
  };
  // checkpoints: first slot of this sequence, half-chunks to the next one
  int ck_slot = 0, ck_next = 0, ck_halves = 1;
  if constexpr (CK) {
    int acc = 0;
    for (int m = lane; m < n; m += 64) {
      const int b0 = min(max(p.cu[m], 0), p.T);
      const int e0 = min(max(p.cu[m + 1], b0), p.T);
      acc += (e0 - b0) / p.ck_int;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    ck_slot = __builtin_amdgcn_readfirstlane(acc);
    ck_halves = p.ck_int / kHT;
    ck_next = ck_halves;
  }
  if (!p.s0) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (p.state_bf16) {
    const uint16_t* s0 = static_cast<const uint16_t*>(p.s0) + sbase + colb;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][rt][j] = bf16_to_f32(s0[key_of(rt, j) * kD + 16 * NSW * u]) * kSDown;
  } else {
    const float* s0 = static_cast<const float*>(p.s0) + sbase + colb;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][rt][j] = s0[key_of(rt, j) * kD + 16 * NSW * u] * kSDown;
  }
  const unsigned cstrip = unsigned(slice * VS + 16 * sw);
  // value rows of a chunk, loaded a chunk ahead into two alternating register
  // sets (no register copies: a copy would wait for the loads, and on gfx9 for
  // the output stores issued before them too).  Past the end: zeros.
  auto load_v = [&](uint2 (&v)[SPW][2], int j) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        v[u][hb] = load_vrow(vsrc, cstrip + 16 * NSW * u, p.ts_v, bos + kC * j + kHT * hb, lane);
  };
  // Per-chunk operands, read from the chunk's package into registers while
  // the previous chunk is computed (the state chain then starts on operands
  // already in registers).
  struct Ops {
    bf16x8 xa[2][4], qa[2][4];  // X^h, Q^h A fragments (row block h, channel block kb)
    bf16x8 la[2], ma[2];        // L / 16, 16 M' A fragments of row block p
    f32x4 bb[2], rr[2];         // b / 16 and scale / |q| of the lane group's tokens
    float2 ga0, ga1;            // Gam_0, Gam_1 factors (gmo order)
  };
  auto load_ops = [&](Ops& o, const Pack& P) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        o.xa[hb][kb] = lds16(&P.x[tro(kHT * hb + l16, 4 * kb + g4)]);
        o.qa[hb][kb] = lds16(&P.qt[tro(kHT * hb + l16, 4 * kb + g4)]);
      }
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      o.la[pb] = lds16(&P.l[pb][8 * lane]);
      o.ma[pb] = lds16(&P.m[pb][8 * lane]);
      o.bb[pb] = *reinterpret_cast<const f32x4*>(&P.b16[kHT * pb + 4 * g4]);
      o.rr[pb] = *reinterpret_cast<const f32x4*>(&P.rqs[kHT * pb + 4 * g4]);
    }
    o.ga0 = *reinterpret_cast<const float2*>(&P.gam[0][2 * lane]);
    o.ga1 = *reinterpret_cast<const float2*>(&P.gam[1][2 * lane]);
  };
  // V rows of a chunk into the accumulator layout (row tile written, read back transposed)
  auto v_acc = [&](const uint2 (&vv)[SPW][2], f32x4 (&V)[SPW][2]) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        Tile& tl = sm.tl[sw][u];
        *reinterpret_cast<uint2*>(&tl.t[hb][4 * lane]) = vv[u][hb];
        __builtin_amdgcn_wave_barrier();
        V[u][hb] = to_f32x4(tr4(&tl.t[hb][4 * lane]));
      }
  };
  // chunk j of slot C in package buffer B (compile-time: every LDS address is
  // a lane offset plus a constant); o holds its operands and receives the
  // next chunk's (slot 1 - C, buffer B ^ C)
  auto chunk = [&](Ops& o, f32x4 (&V)[SPW][2], const uint2 (&vnext)[SPW][2], int j, auto cc, auto bb_) {
    constexpr int c = decltype(cc)::value, bf = decltype(bb_)::value;
    constexpr int cn = c ^ 1, bn = bf ^ c;  // the next chunk's slot and buffer
    const Pack& P = sm.pk[c][bf];
    const Pack& PN = sm.pk[cn][bn];
    const int t0 = bos + kC * j;
    // checkpoints after the first half and after the whole chunk (slots; -1: none)
    int ck_mid = -1, ck_end = -1;
    if constexpr (CK) {
      if (2 * j + 1 == ck_next && kC * j + kHT <= eos - bos) { ck_mid = ck_slot++; ck_next += ck_halves; }
      if (2 * j + 2 == ck_next && kC * (j + 1) <= eos - bos) { ck_end = ck_slot++; ck_next += ck_halves; }
    }
    f32x4 O[SPW][2];
    f16x4 nh[SPW][2];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      // B operands of S (first half) and of Gam_0 S (second half)
      bf16x8 sb[4], s1b[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sb[kb] = cat(to_bf16x4(S[u][2 * kb]), to_bf16x4(S[u][2 * kb + 1]));
      f32x4 Y0 = {0.f, 0.f, 0.f, 0.f}, Q0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Y0 = mfma32(o.xa[0][kb], sb[kb], Y0);
        Q0 = mfma32(o.qa[0][kb], sb[kb], Q0);
      }
      decay_strip(S[u], o.ga0.x, o.ga0.y);  // S <- Gam_0 S
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s1b[kb] = cat(to_bf16x4(S[u][2 * kb]), to_bf16x4(S[u][2 * kb + 1]));
      f32x4 Y1 = {0.f, 0.f, 0.f, 0.f}, Q1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Y1 = mfma32(o.xa[1][kb], s1b[kb], Y1);
        Q1 = mfma32(o.qa[1][kb], s1b[kb], Q1);
      }
      // N / 16 = diag(b / 16) D + (L / 16) D, D = V - Y
      const f32x4 D0 = V[u][0] - Y0, D1 = V[u][1] - Y1;
      const bf16x8 db = cat(to_bf16x4(D0), to_bf16x4(D1));
      const f32x4 N0 = mfma32(o.la[0], db, o.bb[0] * D0);
      const f32x4 N1 = mfma32(o.la[1], db, o.bb[1] * D1);
      // O = rqs (Q S) + (16 M') (N / 16)
      const bf16x8 nbv = cat(to_bf16x4(N0), to_bf16x4(N1));
      O[u][0] = mfma32(o.ma[0], nbv, o.rr[0] * Q0);
      O[u][1] = mfma32(o.ma[1], nbv, o.rr[1] * Q1);
      nh[u][0] = f16x4{(_Float16)N0[0], (_Float16)N0[1], (_Float16)N0[2], (_Float16)N0[3]};
      nh[u][1] = f16x4{(_Float16)N1[0], (_Float16)N1[1], (_Float16)N1[2], (_Float16)N1[3]};
    }
    // this chunk's K' fragments, then (ahead of use, after them in the LDS
    // queue) the next chunk's operands
    f16x4 ka[2][8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
        ka[hb][rt] = tr4h(&P.kp[kpo(kHT * hb + 4 * g4 + (l16 >> 2), rt >> 1, rt & 1, l16 & 3)]);
    const float2 g1 = o.ga1;
    // done with chunk j's package (the K' reads above are complete before the
    // count), before waiting for chunk j + 1: the buffer goes back early
    arrive(&sm.sy.done[c][sw], lane);
    if (j + 1 < nc) {
      const int r1 = (j + 1) >> 1;
      wait_count(&sm.sy.rdy[cn][bn], 4 * ((r1 >> 1) + 1), err);
      load_ops(o, PN);
    }
    // S_mid = Gam_0 S + K'^0T N_0; S <- Gam_1 S_mid + K'^1T N_1 (fp16 K' / 16 and N / 16:
    // 2^-8 of the update, the scale the state is held at)
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[u][rt] = mfma16x(ka[0][rt], nh[u][0], S[u][rt]);
      if constexpr (CK)
        if (ck_mid >= 0 && ck_mid < p.ck_cap) store_strip(p.ck, (size_t(ck_mid) * H + h) * kD * kD, u);
      decay_strip(S[u], g1.x, g1.y);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[u][rt] = mfma16x(ka[1][rt], nh[u][1], S[u][rt]);
      if constexpr (CK)
        if (ck_end >= 0 && ck_end < p.ck_cap) store_strip(p.ck, (size_t(ck_end) * H + h) * kD * kD, u);
    }
    // O to rows: column-major 16x16 tiles (8-byte unit g4 of column l16 at
    // unit g4 ^ (l16 >> 2)), read back transposed, one 8-byte store per lane
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        Tile& tl = sm.tl[sw][u];
        *reinterpret_cast<uint2*>(&tl.t[hb][16 * l16 + 4 * (g4 ^ (l16 >> 2))]) =
            uint2{pkb(O[u][hb][0], O[u][hb][1]), pkb(O[u][hb][2], O[u][hb][3])};
        __builtin_amdgcn_wave_barrier();
        // lane (l16 = token, g4): columns 4 g4 .. + 3 of token l16
        const int col = 4 * g4 + (l16 >> 2);
        const bf16x4 orow = tr4(&tl.t[hb][16 * col + 4 * ((l16 & 3) ^ g4)]);
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u32x2, orow), odst,
            ((unsigned(t0 + kHT * hb) + unsigned(l16)) * unsigned(p.ts_o) + cstrip + 16 * NSW * u + 4u * g4) * 2u,
            0, 0);
      }
    // the next chunk's V in the accumulator layout
    v_acc(vnext, V);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  uint2 va[SPW][2], vb[SPW][2];
  f32x4 V[SPW][2];
  Ops o;
  if (nc > 0) {
    load_v(va, 0);
    wait_count(&sm.sy.rdy[0][0], 4, err);
    load_ops(o, sm.pk[0][0]);
    v_acc(va, V);
  }
  for (int j = 0; j < nc; j += 4) {
    load_v(vb, j + 1);
    chunk(o, V, vb, j, I0{}, I0{});
    if (j + 1 >= nc) break;
    load_v(va, j + 2);
    chunk(o, V, va, j + 1, I1{}, I0{});
    if (j + 2 >= nc) break;
    load_v(vb, j + 3);
    chunk(o, V, vb, j + 2, I0{}, I1{});
    if (j + 3 >= nc) break;
    load_v(va, j + 4);
    chunk(o, V, va, j + 3, I1{}, I1{});
  }
#pragma unroll
  for (int u = 0; u < SPW; ++u) store_strip(p.sT, sbase, u);
  if (lane == 0 && gave_up(err)) p.errword[0] = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

}  // namespace

template <bool CK>
const void* fwd32_fn(int vs, int* threads) {
  switch (vs) {
    case 128: *threads = Cfg32<128>::kThreads; return reinterpret_cast<const void*>(&fwd32_kernel<128, CK>);
    case 64: *threads = Cfg32<64>::kThreads; return reinterpret_cast<const void*>(&fwd32_kernel<64, CK>);
    case 32: *threads = Cfg32<32>::kThreads; return reinterpret_cast<const void*>(&fwd32_kernel<32, CK>);
    case 16: *threads = Cfg32<16>::kThreads; return reinterpret_cast<const void*>(&fwd32_kernel<16, CK>);
    default: return nullptr;
  }
}

hipError_t launch_fwd32(const Params& p, hipStream_t stream) {
  int threads = 0;
  const void* fn = p.ck ? fwd32_fn<true>(kD / p.vsplit, &threads) : fwd32_fn<false>(kD / p.vsplit, &threads);
  if (!fn) return hipErrorInvalidValue;
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(p.N * p.H * p.vsplit), dim3(threads), args, 0, stream);
}

}  // namespace kda
