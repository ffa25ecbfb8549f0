// kda_pipe_parts.h -- pieces shared by the pipelined 16-token kernels
// (kda_pipe.hip: producers and state waves in one workgroup; kda_duo.hip:
// producers and state waves in two workgroups on one XCD): the chunk
// package and its LDS layouts, the producers' loads and their operand,
// inverse and M' steps, the LDS counters and bounded waits, and the
// state-strip helpers.  The method, the exponent ranges and the precision
// plan are described at the top of kda_pipe.hip.
#pragma once

#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kTok = 16;  // tokens per chunk
constexpr int kPH = 2;    // producer waves per chunk (64-channel halves)
constexpr int kSpinMax = 1 << 22;  // polls before a wait gives up (then the status word is set)
constexpr float kKpScale = 16.f;     // K' enters the fp16 state update times this
constexpr float kNScale = 0.0625f;   // ... and N times this (exact inverse)

// [128][16] tiles (row = key channel, column = token; 32 bytes a row, four
// 8-byte token groups).  Row r sits at position p = swz(r) and its token
// group g at slot (g + p / 16) mod 4 of the row.  An 8-byte LDS access serves
// 16 lanes at a time on 32 four-byte banks, so those 16 lanes must cover 16
// distinct (p mod 4, slot) pairs.  The producers' stores (16 rows 4 c + i,
// one token group) get them from the rotation -- without it their 16 rows
// fell on 4 bank pairs, 4-way conflicts, most of the kernel's conflict
// cycles -- and the transposed operand reads (4 consecutive rows x 4 token
// groups) from the row order, which the rotation does not change.
__device__ __forceinline__ int swz(int r) { return r ^ ((r >> 2) & 3); }
__device__ __forceinline__ int tile(int r, int g) {  // element offset of row r, token group g
  const int p = swz(r);
  return p * kTok + 4 * ((g + (p >> 4)) & 3);
}

// Fragment tiles: the A-operand order of a 16x16x16 MFMA.  Element (row m,
// column k) of 16x16 block b sits at (b * 64) + ((k / 4) * 16 + m) * 4 + k % 4,
// so lane (l16, g4) reads its four k-values as 8 contiguous bytes and a wave
// reads one block as 512 contiguous bytes.
__device__ __forceinline__ int frag(int blk, int m, int k) {
  return blk * 256 + ((k >> 2) * 16 + m) * 4 + (k & 3);
}
// The same with the row m of each 8-byte unit permuted by its k group
// (m ^ (k / 4) in the two low bits).  For K' the producers write one key's
// four tokens per lane, and the lanes of a store differ in key only by
// multiples of 4 within their token group: in plain fragment order that puts
// 16 lanes on one bank pair; permuted, the 64 lanes spread over 16.  The
// reader's 512 contiguous bytes per block only change order.
__device__ __forceinline__ int fragx(int blk, int m, int k) {
  return frag(blk, m ^ ((k >> 2) & 3), k);
}

// Buffer resources over one head's rows of a [T, H, ...] tensor, bounded at
// the end of the sequence: loads past it return 0 and stores past it are
// dropped by the hardware range check, so partial chunks need no branches.
// (gfx9 buffer descriptor word 3: 32-bit untyped data.)
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int eos, int rowstride,
                                                          int rowlen) {
  // below 2^32 by the host's size check; formed unsigned
  const unsigned bytes = eos > 0 ? (unsigned(eos - 1) * unsigned(rowstride) + unsigned(rowlen)) * 2u : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcWord3);
}

template <int B>
struct BufIdx {
  static constexpr int value = B;
};

// LDS counters of one workgroup.  A wave's LDS operations complete in order
// and the release below also waits for them, so a wave that observes a count
// (acquire) sees every package write made before the matching increments.
__device__ __forceinline__ void arrive(int* ctr, int lane) {
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *ctr >= target.  Every count a wave waits for is produced by
// waves of the same workgroup that do not wait, directly or through others,
// for the waiting wave, so the wait ends; the poll bound keeps a broken count
// from holding the device, and giving up is recorded in the LDS word err
// (every later wait then returns at once, so all waves finish quickly, and
// the kernel reports it in the workspace's status word).
__device__ __forceinline__ bool gave_up(const int* err) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
}
__device__ __forceinline__ void wait_count(const int* ctr, int target, int* err) {
  if (gave_up(err)) return;
#pragma unroll 1
  for (int it = 0; it < kSpinMax; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One chunk's package: written by the chunk's two producer waves, read by
// the state waves.
struct Pack {
  bf16 x[128 * kTok];    // X = e^{G} k~, swizzled rows
  bf16 qt[128 * kTok];   // Q_T = e^{G} q, swizzled rows
  bf16 kp[128 * kTok];   // kKpScale K' as fp16, permuted fragment order (fragx; block = 16 keys)
  bf16 l[256];           // L, fragment order
  bf16 m[256];           // M', fragment order
  float beta[kTok];
  float rqs[kTok];       // scale / ||q_t||
  float rk[kPH][kTok];   // 1 / ||k_t||, one copy per producer wave (scratch)
  float gam[128];        // e^{G_last}
};
static_assert(sizeof(Pack::gam) >= sizeof(int) * (kInlineRankMax + 1), "rank scratch fits in gam");
static_assert(sizeof(Pack) % 16 == 0, "packages stay 16-byte aligned");

// Raw inputs of one chunk for one producer lane of channel half hf: tokens
// 4 tq + rr (rr = 0..3) of channels 64 hf + 4 cg .. + 3 (cg = lane % 16,
// tq = lane / 16, so each load instruction reads four 128-byte row segments,
// 16 consecutive lanes each); k again as rows for its norm (token lane / 4,
// channels 32 (lane % 4) ..); for the second half q as rows as well, for the
// first the beta logit of token `lane` (lanes < 16).
struct Raw {
  uint2 q[4], k[4], g[4];
  uint4 kn[4], qn[4];
  uint32_t beta;
};

// Head h's rows, bounded at the sequence end.  qn and beta: the q rows for
// the second channel half, the beta logits for the first; the other half gets
// an empty resource (its loads return zeros without touching memory), so the
// loads need no branch (a branch here makes the compiler copy, and so wait
// for, the loaded registers).
struct RawSrc {
  __amdgpu_buffer_rsrc_t q, k, g, qn, beta;
};

// Loads of one chunk's raw inputs, in three groups so that a chunk's loads
// can be issued while the previous chunk's operands are formed, each group as
// soon as its registers have been consumed.  Rows past the sequence end read
// as zeros (buffer range check), so the loads need no condition.
struct RawLoad {
  RawSrc src;
  int ts_q, ts_k, ts_g, ts_b, lane, hf;  // token strides (elements) of q, k, g, beta

  // rows for the norms, and beta
  __device__ __forceinline__ void rows(Raw& r, int t0) const {
    const unsigned tok = unsigned(t0) + unsigned(lane >> 2), c0 = 32u * unsigned(lane & 3);
    const unsigned offk = (tok * unsigned(ts_k) + c0) * 2u, offq = (tok * unsigned(ts_q) + c0) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.kn[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src.k, offk + 16u * i, 0, 0));
      if (hf) r.qn[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src.qn, offq + 16u * i, 0, 0));
    }
    if (!hf) r.beta = __builtin_amdgcn_raw_buffer_load_b16(src.beta, (unsigned(t0) + unsigned(lane)) * unsigned(ts_b) * 2u, 0, 0);
  }
  __device__ __forceinline__ unsigned col_off(int t0, int rr, int ts) const {
    const unsigned ch = 64u * unsigned(hf) + 4u * unsigned(lane & 15), tq = unsigned(lane >> 4);
    return ((unsigned(t0) + 4u * tq + rr) * unsigned(ts) + ch) * 2u;
  }
  // gate inputs
  __device__ __forceinline__ void gate(Raw& r, int t0) const {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      r.g[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.g, col_off(t0, rr, ts_g), 0, 0));
  }
  // q and k
  __device__ __forceinline__ void qk(Raw& r, int t0) const {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      r.q[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.q, col_off(t0, rr, ts_q), 0, 0));
      r.k[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src.k, col_off(t0, rr, ts_k), 0, 0));
    }
  }
  // in the loop's issue order (gate, rows, q/k), which the scheduler must
  // keep: the waits at the top of the loop are computed over both ways in,
  // so a different order here would make the first waits of every round
  // drain the whole queue
  __device__ __forceinline__ void all(Raw& r, int t0) const {
    gate(r, t0);
    __builtin_amdgcn_sched_barrier(0);
    rows(r, t0);
    __builtin_amdgcn_sched_barrier(0);
    qk(r, t0);
  }
};

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

// Value of another lane of the same quad (DPP quad_perm pattern CTRL).
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Lane N of this lane's row of 16 (DPP row_newbcast; the backend folds it
// into the consuming VALU instruction).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

// Sum over the four lanes of a quad.
__device__ __forceinline__ float quad_sum(float s) {
  s += quad_perm<0xB1>(s);  // [1,0,3,2]
  s += quad_perm<0x4E>(s);  // [2,3,0,1]
  return s;
}

// sum over the row of 32 channels held by each lane of a quad
__device__ __forceinline__ float row_norm2(const uint4* w) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = dot2(w[i].x, s);
    s = dot2(w[i].y, s);
    s = dot2(w[i].z, s);
    s = dot2(w[i].w, s);
  }
  return quad_sum(s);
}

// Channel i (0..3) of a 4-channel bf16 group.
__device__ __forceinline__ float chan(uint2 w, int i) {
  const uint32_t d = i < 2 ? w.x : w.y;
  return (i & 1) ? bf16_hi(d) : bf16_lo(d);
}

// Producer, first phase (both waves of a chunk, one channel half each): the
// norm of k (and of q, or beta), the gate and its cumulative sum, and every
// decayed operand of the half's 64 channels.  Writes X = e^G k~ and Q_T =
// e^G q, the products' right operand K_G = e^{-G} k~ (to `kg`), kKpScale K'
// (fp16), gam, and rqs (second half) or beta (first half).  FULL: all 16
// tokens are inside the sequence (no masking).  NOQ: no output is formed
// (the summary step), so neither Q_T nor rqs.
template <bool FULL, bool NOQ = false>
__device__ __forceinline__ void produce_operands(Pack& pk, bf16* kg, Raw& raw,
                                                 const RawLoad& ld, int tn, int hf, int Lc, int lane,
                                                 const float* c2, float c1, float lb2, float scale) {
  const int cg = lane & 15, tq = lane >> 4;

  // gate sigma per (token, channel), its running sum over this lane's 4
  // tokens, then the sum over the earlier token groups (lanes 16 apart, by
  // lane permutes); the log2 decay of a token is lb2 * sigma (lb2 =
  // lower_bound log2 e)
  float cs[4][4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const bool valid = FULL || 4 * tq + rr < Lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sg = rcp(1.f + ex2(fmaf(chan(raw.g[rr], i), c1, c2[i])));
      const float inc = valid ? sg : 0.f;
      cs[i][rr] = rr == 0 ? inc : cs[i][rr - 1] + inc;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the next chunk's gate inputs (tn), into the registers just consumed:
  // they are the first thing the next round needs, so they get the longest lead
  ld.gate(raw, tn);
  __builtin_amdgcn_sched_barrier(0);
  // 1 / ||k_t|| and scale / ||q_t|| or beta_t for token lane/4 (beta: lane)
  {
    const float sk = row_norm2(raw.kn);
    if ((lane & 3) == 0) pk.rk[hf][lane >> 2] = rsqrtf(sk + kNormEps);
    if (hf) {
      if constexpr (!NOQ) {
        const float sq = row_norm2(raw.qn);
        if ((lane & 3) == 0) pk.rqs[lane >> 2] = rsqrtf(sq + kNormEps) * scale;
      }
    } else if (lane < kTok) {
      pk.beta[lane] = lane < Lc ? rcp(1.f + ex2(-kLog2e * bf16_to_f32(uint16_t(raw.beta)))) : 0.f;
    }
  }
  // the next chunk's rows (tn), into the registers just consumed
  __builtin_amdgcn_sched_barrier(0);
  ld.rows(raw, tn);
  __builtin_amdgcn_sched_barrier(0);

  // the 4-token totals of the other token groups of this channel (rows of 16
  // lanes): permlane16_swap gives each lane its row pair's even and odd row,
  // permlane32_swap the two pairs' sums; no LDS round trip
  float off[4], gam[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned t = __float_as_uint(cs[i][3]);
    const auto pr = __builtin_amdgcn_permlane16_swap(t, t, false, false);
    const float te = __uint_as_float(pr[0]), to = __uint_as_float(pr[1]);  // rows tq & ~1, tq | 1
    const unsigned pp = __float_as_uint(te + to);
    const auto pq = __builtin_amdgcn_permlane32_swap(pp, pp, false, false);
    const float p01 = __uint_as_float(pq[0]), p23 = __uint_as_float(pq[1]);  // rows 0 + 1, 2 + 3
    const float excl = ((tq & 2) ? p01 : 0.f) + ((tq & 1) ? te : 0.f);      // groups before tq
    off[i] = lb2 * excl;
    gam[i] = ex2(lb2 * (p01 + p23));  // e^{G_last}
  }
  if (tq == 0)
    *reinterpret_cast<f32x4*>(&pk.gam[64 * hf + 4 * cg]) = f32x4{gam[0], gam[1], gam[2], gam[3]};

  // 1 / ||k|| of this lane's 4 tokens (written above by other lanes of this wave)
  __builtin_amdgcn_wave_barrier();
  const f32x4 rk4 = *reinterpret_cast<const f32x4*>(&pk.rk[hf][4 * tq]);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 64 * hf + 4 * cg + i;
    const int row = tile(c, tq);  // this lane's 4 tokens of channel c
    const float g16 = kKpScale * gam[i];
    float vx[4], vq[4], vg[4], vk[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float G = fmaf(cs[i][rr], lb2, off[i]);
      const float E = ex2(G), F = ex2(-G);
      const float kv = chan(raw.k[rr], i) * rk4[rr];
      vx[rr] = kv * E;
      if constexpr (!NOQ) vq[rr] = chan(raw.q[rr], i) * E;
      vg[rr] = kv * F;
      vk[rr] = vg[rr] * g16;
    }
    *reinterpret_cast<uint2*>(&pk.x[row]) = uint2{pk2(vx[0], vx[1]), pk2(vx[2], vx[3])};
    if constexpr (!NOQ) *reinterpret_cast<uint2*>(&pk.qt[row]) = uint2{pk2(vq[0], vq[1]), pk2(vq[2], vq[3])};
    *reinterpret_cast<uint2*>(&kg[row]) = uint2{pk2(vg[0], vg[1]), pk2(vg[2], vg[3])};
    *reinterpret_cast<uint2*>(&pk.kp[fragx(c >> 4, c & 15, 4 * tq)]) =
        uint2{pk2h(vk[0], vk[1]), pk2h(vk[2], vk[3])};
  }
  __builtin_amdgcn_sched_barrier(0);
  ld.qk(raw, tn);
}

// Producer, second phase, first wave of a chunk: A = X K_G^T and A^T over the
// 128 channels, the inverse (I + A)^-1 and L.
__device__ __forceinline__ void produce_inverse(Pack& pk, const bf16* kg, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;

  // k-slots 8 g4 .. 8 g4 + 7 of each 32-channel block, on both sides
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 accA = zero, accAt = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int r1 = 32 * kb + 8 * g4 + (l16 >> 2), r2 = r1 + 4;
    const int o1 = tile(r1, l16 & 3), o2 = tile(r2, l16 & 3);
    const bf16x8 KE = cat(tr4(&pk.x[o1]), tr4(&pk.x[o2]));
    const bf16x8 KG = cat(tr4(&kg[o1]), tr4(&kg[o2]));
    accA = mfma32(KE, KG, accA);     // [t = 4g4+j][i = l16]
    accAt = mfma32(KG, KE, accAt);   // [i = 4g4+j][t = l16]
  }

  const f32x4 bR = *reinterpret_cast<const f32x4*>(&pk.beta[4 * g4]);
  const float bC = pk.beta[l16];
  f32x4 Nn, Nt, I4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g4 + j;
    Nn[j] = l16 < r ? bR[j] * accA[j] : 0.f;    // A[r][l16]
    Nt[j] = r < l16 ? bC * accAt[j] : 0.f;      // A[l16][r]
    I4[j] = r == l16 ? 1.f : 0.f;
  }

  // (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) (A^16 = 0).  Each product is
  // formed together with its transpose: an accumulator holds Z[4g+j][l16],
  // which is Z's B-operand layout and Z^T's A-operand layout, so Z = X Y is
  // mfma(X^T, Y) and Z^T = Y^T X^T is mfma(Y, X^T).
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

// Producer, second phase, second wave of a chunk: M' = rqs (Q_T K_G^T).
__device__ __forceinline__ void produce_m(Pack& pk, const bf16* kg, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  f32x4 accMt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int r1 = 32 * kb + 8 * g4 + (l16 >> 2), r2 = r1 + 4;
    const int o1 = tile(r1, l16 & 3), o2 = tile(r2, l16 & 3);
    const bf16x8 KG = cat(tr4(&kg[o1]), tr4(&kg[o2]));
    const bf16x8 QE = cat(tr4(&pk.qt[o1]), tr4(&pk.qt[o2]));
    accMt = mfma32(KG, QE, accMt);   // [i = 4g4+j][t = l16]
  }
  const float rqC = pk.rqs[l16];
  f32x4 Mv;
#pragma unroll
  for (int j = 0; j < 4; ++j) Mv[j] = 4 * g4 + j <= l16 ? rqC * accMt[j] : 0.f;   // M'[l16][4g4+j]
  *reinterpret_cast<bf16x4*>(&pk.m[frag(0, l16, 4 * g4)]) = to_bf16x4(Mv);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// S <- Diag(e^{G_last}) S on one state strip in the accumulator layout (lane
// (l16, g4) holds rows 16 rt + 4 g4 + j).  Each lane has read two of its
// row's 32 factors, g[16 (l16 / 2) + 4 g4 + 2 (l16 % 2) + {0, 1}], so row rt,
// element j sits in lane 2 rt + j / 2 of the same 16 (component j % 2): one
// 8-byte LDS read per lane instead of eight 16-byte ones, and the broadcast
// rides on the multiply.
template <int RT = 0>
__device__ __forceinline__ void decay_strip(f32x4 (&S)[8], float g0, float g1) {
  S[RT][0] = S[RT][0] * row_bcast<2 * RT>(g0);
  S[RT][1] = S[RT][1] * row_bcast<2 * RT>(g1);
  S[RT][2] = S[RT][2] * row_bcast<2 * RT + 1>(g0);
  S[RT][3] = S[RT][3] * row_bcast<2 * RT + 1>(g1);
  if constexpr (RT < 7) decay_strip<RT + 1>(S, g0, g1);
}
// Value strip (16 tokens x 16 columns) of one chunk as rows: lane L holds
// columns 4 (L % 4) .. + 3 of token L / 4, one 8-byte load (zero past the
// sequence end).
__device__ __forceinline__ uint2 load_vrow(__amdgpu_buffer_rsrc_t v, unsigned c0, int rowstride,
                                           int t0, int lane) {
  const unsigned off =
      ((unsigned(t0) + unsigned(lane >> 2)) * unsigned(rowstride) + c0 + 4u * unsigned(lane & 3)) * 2u;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(v, off, 0, 0));
}

// Per state wave and strip: 16 x 16 bf16 tiles that turn the row-wise value
// loads into the accumulator layout and the output back into rows, so global
// memory sees 8-byte accesses only.
struct Tiles {
  bf16 v[256];  // V rows, row-major [token][column]
  bf16 o[256];  // O, column-major [column][token]
};

// Wait until the first n counters of a 16-byte row are all >= target: one
// LDS read per poll (same bound and argument as wait_count).  Used before
// overwriting what the counting waves have read: their release made those
// reads complete, the caller's writes are issued only after the exit branch
// (which waits for the value), and the compiler barrier keeps them there.
template <int n>
__device__ __forceinline__ void wait_row(const int* row, int target, int* err) {
  if (gave_up(err)) return;
#pragma unroll 1
  for (int it = 0; it < kSpinMax; ++it) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
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
  __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace
}  // namespace kda
