// kda_internal.h -- shared definitions of the gfx950 KDA kernels and the host
// library that launches them.  Not part of the public ABI (include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;  // head_dim (keys and values)
constexpr float kNormEps = 1e-6f;

// Everything a kernel needs for one call.  Tensor layouts are those of
// include/kda.h: q/k/v/g/out [T, H, D] bf16 rows at the strides below, beta
// [T, H] bf16, state [N, H, D, D] (row = key channel, column = value channel).
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  const void* s0;  // may be null (zeros)
  void* sT;
  uint16_t* out;
  const int32_t* cu;
  int32_t* order;  // sequence processing order (longest first), [N], in the workspace;
                   // null: the kernel ranks the sequences itself (pipelined kernels, N small)
  int32_t* errword;  // the workspace's status word: a kernel sets it (nonzero) if a
                     // bounded wait gave up (never cleared here)
  float lower_bound;
  float scale;
  // element strides of the per-token tensors (channels contiguous): row
  // (t, h) of q starts at q + t * ts_q + h * hs_q; beta[t, h] at
  // beta + t * ts_b + h * hs_b.  Every (T + 256) * ts + (H - 1) * hs + 128 < 2^31.
  int ts_q, ts_k, ts_v, ts_g, ts_b, ts_o;
  int hs_q, hs_k, hs_v, hs_g, hs_b, hs_o;
  int T;           // tokens in q/k/v/g/out (sequence offsets are clamped to it)
  int H;
  int N;
  int vsplit;      // value-dimension slices per (sequence, head)
  int state_bf16;  // 0: fp32 state, 1: bf16 state
  // checkpoint states (pipelined kernel only): null, or [ck_cap, H, D, D] in
  // the state dtype, one after every ck_int tokens of each sequence
  void* ck;
  int ck_int;
  int64_t ck_cap;
  // speculative-decode step (token-serial kernels only): null, or [N, sp_stride]
  // state slots; sequence n starts from slot sp_idx[n][sp_acc[n] - 1] of the
  // pool (s0 = sT = the pool, [sp_slots, H, D, D]) and stores the state after
  // its t-th token in slot sp_idx[n][t].  Slots outside [0, sp_slots) read as
  // the zero state and are not written; so are accepted counts outside
  // [1, sp_stride] and tokens past sp_stride.
  const int32_t* sp_idx;
  const int32_t* sp_acc;
  int sp_stride;
  int64_t sp_slots;
  // segment-parallel schedule (pipelined 16-token kernel only): null, or one
  // entry of four ints per pseudo-sequence m = 0 .. N - 1 of the grid (N is
  // then the entry count): the sequence n (-1: unused entry, the workgroup
  // exits), its first and end token, flags (bit 0: n's last segment).
  //   seg_mode 1, summaries: the slices cover 256 columns, the local state
  //     (values v, from zero) and the transition (values 0, from the
  //     identity); outputs are not written; both go to sT = [N, H, 2, D, D]
  //     fp32 at m.  Last segments have no summary (they exit).
  //   seg_mode 2, rerun: the initial state is s0 = [N, H, D, D] fp32 at m;
  //     the final state goes to sT at sequence n, in the state dtype, for
  //     last segments only.
  const int32_t* seg;
  int seg_mode;
  // two-workgroup forward (kda_duo.hip): per item, kDuoRing chunk packages of
  // kDuoPkgBytes (duo_ring) and kDuoFlagWords flag words (duo_flags);
  // duo_nonce marks this call's flag words
  void* duo_ring;
  uint64_t* duo_flags;
  uint32_t duo_nonce;
};

// The two-workgroup forward: packages per item in flight between its two
// workgroups, and their size in the workspace (a package rounded up to 1 KB).
constexpr int kDuoRing = 4;
constexpr int kDuoPkgBytes = 14336;
constexpr int kDuoFlagWords = 8;  // uint64 flag words per (sequence, head)

// Pseudo-sequences of the segment-parallel schedule (kda_segment.hip).  Each
// sequence n is cut into count[n] = max(1, ceil(len / L)) segments of L tokens
// (the last shorter), pseudo-sequences first[n] .. first[n] + count[n] - 1.
struct SegParams {
  const int32_t* cu;  // [N + 1] sequence offsets (clamped like the kernels do)
  int N, T, H, L;
  int M;              // table entries (the grid's pseudo-sequences), >= N + T / L
  int32_t* table;     // [M][4]: n (or -1), first token, end token, flags (bit 0: last)
  int32_t* first;     // [N]
  int32_t* count;     // [N]
  const void* s0;     // the caller's initial state [N, H, D, D] (null: zeros)
  int s0_bf16;
  const float* summ;  // [M, H, 2, D, D]: local state, transition
  float* starts;      // [M, H, D, D]: the state entering each pseudo-sequence
};
// The table (one workgroup).
hipError_t launch_seg_plan(const SegParams& sp, hipStream_t stream);
// The states entering every segment: S_0 = the initial state, S_{j+1} =
// P_j S_j + R_j in fp32, one workgroup per (sequence, head, 16 columns).
hipError_t launch_seg_combine(const SegParams& sp, hipStream_t stream);

// ---- bf16 helpers (bf16 is the high half of an IEEE fp32) -------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Workgroup index B of a grid of G -> work item b = rank * s + slice (s value
// slices per (sequence rank, head) item).  The dispatcher hands workgroups to
// the 8 XCDs round robin (B on XCD (B + o) mod 8; the offset o depends on where
// the previous dispatch ended), so items are handed out in rank order across
// the XCDs (ranked, longest-first work spreads evenly over them) and the s
// slices of one item sit on one XCD, 8 workgroup indices apart, sharing q/k/g
// in its L2.  Identity when G is not a multiple of 8 s.
__device__ __forceinline__ int work_item(int B, int G, int s) {
  if (G % (8 * s)) return B;
  const int xcd = B & 7, k = B >> 3;
  return ((k / s) * 8 + xcd) * s + k % s;
}

// ---- launch entry points (one per kernel family) -----------------------------

// Sequence order, longest first (ties by index), into p.order.  One launch.
hipError_t launch_plan(const Params& p, hipStream_t stream);

// Token-serial fp32 recurrence, one workgroup per (sequence, head, V-slice).
// decode: the decode kernel (16-byte state accesses, 4 tokens staged at a
// time; slices of 16 or 32 columns stage 4 tokens in the 4-byte kernel), for
// sequences of a few tokens, giving the same bits.  p.order may be null
// (sequences taken in index order).
hipError_t launch_recurrent(const Params& p, hipStream_t stream, bool decode);

// Chunked (64-token WY/UT) forward with bf16 MFMA, one workgroup per
// (sequence, head, V-slice).
hipError_t launch_chunk(const Params& p, hipStream_t stream);

// Pipelined 16-token chunk forward: producer waves build each chunk's
// state-independent operands ahead of the state waves, one workgroup per
// (sequence, head, V-slice).  Requires lower_bound >= kPipeLowerBoundMin and a
// value slice of at most 64 columns (vsplit >= 2).
// With at most kInlineRankMax sequences it ranks them itself (p.order may be
// null and no plan launch is needed).
constexpr float kPipeLowerBoundMin = -5.0f;
// Calls with at most this many tokens per sequence on average go to the
// token-serial kernel with decode staging.
constexpr int kDecodeTokensPerSeq = 8;
constexpr int kInlineRankMax = 16;
hipError_t launch_pipe(const Params& p, hipStream_t stream);

// The same 16-token forward with the producers and the state waves in two
// workgroups of one XCD per (sequence, head): 2 * 8 ceil(N H / 8) workgroups,
// which must all fit on the device at once (2 N H <= CUs); all 128 value
// columns in one workgroup, the packages through p.duo_ring, p.duo_flags
// (N H entries each) and the call's p.duo_nonce.  Lower bound as above.
hipError_t launch_duo(const Params& p, hipStream_t stream);

// Pipelined 32-token chunk forward (two 16-token halves with their own decay
// reference points): four producer waves build the packages of alternating
// chunks, the state waves walk them in order.  Any value slice of 16..128
// columns, lower_bound in [-5.5, 0].  Ranks up to kInlineRankMax sequences
// itself.
hipError_t launch_fwd32(const Params& p, hipStream_t stream);

// ---- the gate / beta projections (kda_proj.hip) ---------------------------------
constexpr int kProjRank = 128;  // inner dimension of the gate's second factor
// Row-major bf16 matrices: hidden [M, K], w_ab [n_ab, K], w_b [n_b, 128];
// outputs p_ab [M, n_ab], g [M, n_b].  partials: the workspace
// (proj_workspace_bytes), written before it is read in every call.
struct ProjParams {
  const uint16_t* hidden;
  const uint16_t* w_ab;
  const uint16_t* w_b;
  uint16_t* p_ab;
  uint16_t* g;
  float* partials;
  int M, K, n_ab, n_b;
};
size_t proj_workspace_bytes(int M, int K, int n_ab);
// Two launches: P = bf16(hidden w_ab^T), then G = bf16(P[:, :128] w_b^T).
hipError_t launch_proj(const ProjParams& p, hipStream_t stream);

}  // namespace kda
