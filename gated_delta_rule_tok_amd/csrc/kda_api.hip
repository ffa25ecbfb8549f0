// kda_api.hip -- the C ABI of libkda.so (declared in include/kda.h): argument
// checks, workspace sizing, value-split planning and the launches.
//
// The interface mirrors the FlashKDA wrapper in vLLM PR #55737's report
// ("Key source snippets": a workspace-size query taking
// (max_num_batched_tokens, local_num_heads, max_num_seqs), and a forward call
// taking q, k, v, g, raw beta, scale, out, workspace, A_log, dt_bias,
// lower_bound, initial_state, final_state, cu_seqlens), with the sizes, the
// state dtype and the workspace capacity added so a C caller can be checked.
// Failing fast on a bad configuration follows the same page's backend
// resolver ("Implementation breakdown", item 1).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

std::atomic<int> g_vsplit_override{0};
std::atomic<int> g_kernel_override{0};
std::atomic<int> g_segment_override{0};
std::atomic<int> g_cu_count[kMaxDevices];

thread_local char t_last_hip_error[256] = "";

// Scratch of kda_chunk_prefill_fwd_noalloc (for callers that cannot
// allocate): the sequence order table, kNoAllocMaxSeqs entries, one copy per
// device for the life of the process.  Host code never uses the array's name
// as an address: its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int kNoAllocMaxSeqs = 65536;
static __device__ __align__(256) int32_t scratch[kNoAllocMaxSeqs];
std::atomic<int32_t*> g_scratch[kMaxDevices];

hipError_t scratch_address(int32_t** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch));
        e != hipSuccess)
      return e;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The integer a C caller passed for an enum parameter, read without loading it
// as the enum type (a value outside the enumerators is then no undefined
// behaviour, just an invalid argument).
template <typename E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum parameters are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

kda_status_t hip_failure(hipError_t e, const char* step) {
  std::snprintf(t_last_hip_error, sizeof t_last_hip_error, "%s (%s) during %s", hipGetErrorName(e),
                hipGetErrorString(e), step);
  return KDA_ERR_HIP;
}

// Compute units of the current device (cached per device; no synchronisation).
hipError_t device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return hipSuccess;
}

// Value-dimension split (PR #52458's report, "Features and motivation": split
// the value dimension when 2 * heads * sequences <= SM count, i.e. when the
// unsplit pass would leave at least half the machine idle).  Doubling goes on
// while the doubled grid still fits in one wave of workgroups, down to 16
// value columns per workgroup.
int plan_vsplit(int heads, int seqs, int cus) {
  int s = 1;
  const int64_t pairs = int64_t(heads) * seqs;
  while (s < 8 && 2 * s * pairs <= cus) s *= 2;
  return s;
}

// ---- the segment-parallel schedule (kda_segment.hip) ---------------------------
// Long sequences in a call with few (sequence, head) items are cut into
// segments that run in parallel.  Taken when there are at most
// kSegItemsMax items, at least kSegMinAvg tokens per sequence on average
// (twice that with more than kSegItemsMax / 2 items) and the workspace holds
// the segment area.  The segment length aims at about
// kSegTarget / heads segments in the call (so summaries and reruns fill the
// machine), at least kSegMinLen tokens, a multiple of 64 (whole rounds of
// four 16-token chunks).  Measured over shapes of 1-8 sequences of
// 512-65536 tokens and 2-32 heads: at 1024 tokens per sequence 256-token
// segments gain about 12% and 512-token ones lose (with 32 items every cut
// loses there), at 512 tokens every cut loses; 64 items would fill the
// machine with plain workgroups already.
constexpr int kSegItemsMax = 32;
constexpr int64_t kSegMinAvg = 1024;
constexpr int kSegTarget = 128;
constexpr int kSegMinLen = 256;

// Pseudo-sequences a call may use: a call that takes the schedule has at
// most kSegItemsMax / heads sequences and kSegTarget / heads + its sequence
// count segments, so pseudo-sequences x heads <= kSegSlots.
constexpr int kSegSlots = kSegItemsMax + kSegTarget;

// ---- the two-workgroup forward (kda_duo.hip) ------------------------------------
// A producer and a consumer workgroup per (sequence, head) item, all of them
// on the device at once: taken for more than kDuoItemsMin and at most
// kDuoItemsMax items with 2 items <= CUs (where the single-workgroup kernel
// splits the values and repeats each item's state-independent work), above
// kDuoItemsAny items only up to kDuoWorkMax (token, head) pairs in the call,
// when the workspace holds the segment area (the package rings and flag
// words live there).  Measured over 32-128 items of 128-4096 tokens: faster
// or equal up to 96 items at every length (64 items x 4096 tokens 240
// against 248 us, 96 x 2048 124 against 130) and above that for short
// sequences (128 x 1024 69 against 72, 128 x 512 41 against 46, 128 x 256
// 27 against 31), slower for 112-128 items of 2048 tokens (145 against 135,
// 151 against 140: the packages' L2 traffic there costs more than the
// repeated producer work).
constexpr int kDuoItemsMin = 32;
constexpr int kDuoItemsAny = 96;
constexpr int kDuoItemsMax = 128;
constexpr int64_t kDuoWorkMax = int64_t(1) << 17;
std::atomic<uint32_t> g_duo_nonce{0x2545f491u};

// Whether a call of the 16-token family with the workspace's second part
// takes the two-workgroup form (forced: on request, kernel 6).
bool duo_rule(int64_t T, int heads, int seqs, int cus, bool forced) {
  const int64_t items = int64_t(seqs) * heads;
  if (items <= 0 || items > kDuoItemsMax || 2 * items > cus) return false;
  return forced || (items > kDuoItemsMin && (items <= kDuoItemsAny || T * heads <= kDuoWorkMax));
}
int seg_cap(int heads) { return heads <= kSegItemsMax ? kSegSlots / heads : 0; }

// The segment area, one size for every head count (so the workspace size
// stays monotone): the table, first and count arrays for up to kSegSlots
// pseudo-sequences, and kSegSlots (pseudo-sequence, head) slots of summaries
// (local state, transition) and entering states, fp32 128 x 128 each.
struct SegLayout {
  size_t table, first, count, summ, starts, duo_flags, bytes;
};
constexpr size_t kDD = size_t(KDA_HEAD_DIM) * KDA_HEAD_DIM * sizeof(float);
SegLayout seg_layout() {
  SegLayout l{};
  l.table = 0;
  l.first = l.table + align_up(16 * size_t(kSegSlots));
  l.count = l.first + align_up(4 * size_t(kSegSlots));
  l.summ = l.count + align_up(4 * size_t(kSegSlots));
  l.starts = l.summ + size_t(kSegSlots) * 2 * kDD;
  l.duo_flags = l.starts + size_t(kSegSlots) * kDD;
  l.bytes = l.duo_flags + align_up(kda::kDuoFlagWords * sizeof(uint64_t) * size_t(kDuoItemsMax));
  return l;
}
// The two-workgroup forward's package rings share the space of the
// summaries and entering states (a call takes one schedule or the other).
static_assert(size_t(kDuoItemsMax) * kda::kDuoRing * kda::kDuoPkgBytes <= size_t(kSegSlots) * 3 * kDD,
              "the package rings fit in the summaries' and entering states' space");

// Status word and the sequence order table.
size_t base_workspace_bytes(int32_t seqs) { return kAlign + align_up(sizeof(int32_t) * size_t(seqs)); }

// Segment length of a call, or 0 for the plain schedule.  forced: the test
// hook (0 automatic, 1 never, else that length).
int plan_segment_len(int64_t T, int heads, int seqs, int forced) {
  const int cap = seg_cap(heads);
  if (forced == 1 || cap == 0 || T == 0) return 0;
  int64_t L;
  if (forced > 1) {
    L = forced;
  } else {
    const int64_t items = int64_t(seqs) * heads;
    if (items > kSegItemsMax || T < kSegMinAvg * seqs * (2 * items > kSegItemsMax ? 2 : 1)) return 0;
    const int64_t target = kSegTarget / heads;
    L = (T + target - 1) / target;
    L = std::max<int64_t>(kSegMinLen, (L + 63) / 64 * 64);
  }
  if (seqs + T / L > cap) return 0;
  return int(L);
}

}  // namespace

extern "C" {

size_t kda_get_workspace_size(int64_t max_tokens, int32_t heads, int32_t max_seqs) {
  if (max_tokens < 0 || heads <= 0 || max_seqs <= 0) return 0;
  // status word (padded to kAlign), the sequence order table (longest first),
  // and, where some call within these bounds may take the segment-parallel
  // schedule, its area (independent of the token and sequence counts)
  const size_t seg = max_tokens >= kSegMinAvg ? seg_layout().bytes : 0;
  return base_workspace_bytes(max_seqs) + seg;
}

const char* kda_status_string(kda_status_t status) {
  switch (enum_value(status)) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null pointer, bad size or bad scalar";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: lower_bound outside the supported range";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_hip_error(void) { return t_last_hip_error; }

int kda_debug_set_kernel(int k) {
  // 0 automatic, 1 64-token chunk, 2 token-serial, 3 token-serial decode
  // staging (4 tokens), 4 pipelined 16-token in one workgroup per item, 5
  // pipelined 32-token, 6 pipelined 16-token in two workgroups per item
  if (k < 0 || k > 6) return -1;
  return g_kernel_override.exchange(k);
}

int kda_debug_set_segment(int len) {
  // 0 automatic, 1 never, else force segments of len tokens (a multiple of 16)
  if (!(len == 0 || len == 1 || (len >= 16 && len % 16 == 0 && len <= (1 << 24)))) return -1;
  return g_segment_override.exchange(len);
}

int32_t kda_debug_segment_length(int64_t num_tokens, int32_t heads, int32_t num_seqs) {
  if (num_tokens < 0 || heads <= 0 || num_seqs <= 0) return 0;
  return plan_segment_len(num_tokens, heads, num_seqs, g_segment_override.load(std::memory_order_relaxed));
}

int32_t kda_debug_two_workgroups(int64_t num_tokens, int32_t heads, int32_t num_seqs, int32_t cus) {
  if (num_tokens < 0 || heads <= 0 || num_seqs <= 0 || cus <= 0) return 0;
  const int k = g_kernel_override.load(std::memory_order_relaxed);
  if (g_vsplit_override.load(std::memory_order_relaxed) != 0 || !(k == 0 || k == 4 || k == 6)) return 0;
  if (k != 6 && num_tokens <= kda::kDecodeTokensPerSeq * int64_t(num_seqs)) return 0;  // decode-sized
  if (k != 6 && plan_segment_len(num_tokens, heads, num_seqs,
                                 g_segment_override.load(std::memory_order_relaxed)) > 0)
    return 0;  // the segment-parallel schedule comes first
  return duo_rule(num_tokens, heads, num_seqs, cus, k == 6) ? 1 : 0;
}

int kda_debug_set_vsplit(int s) {
  if (!(s == 0 || s == 1 || s == 2 || s == 4 || s == 8)) return -1;
  return g_vsplit_override.exchange(s);
}

}  // extern "C"

namespace {

// Stride checks of one [T, H, 128] tensor: non-negative multiples of 8
// elements, and every row up to 256 past the end addressable with 32-bit
// byte offsets.  Each product and sum is checked for overflow (a caller's
// stride near 2^63 must not wrap into range).
bool rows_ok(int64_t ts, int64_t hs, int64_t T, int64_t H, int64_t rowlen, int64_t align) {
  if (ts < 0 || hs < 0 || ts % align || hs % align) return false;
  if (ts > INT32_MAX || hs > INT32_MAX) return false;
  int64_t rows = 0, heads = 0, end = 0;
  if (__builtin_mul_overflow(T + 256, ts, &rows) || __builtin_mul_overflow(H - 1, hs, &heads) ||
      __builtin_add_overflow(rows, heads, &end) || __builtin_add_overflow(end, rowlen, &end))
    return false;
  return end <= INT32_MAX;
}

kda_status_t forward(const void* q, const void* k, const void* v, const void* g,
                     const void* beta_logits, const float* A_log, const float* dt_bias,
                     float lower_bound, float scale, const void* initial_state,
                     const int32_t* cu_seqlens, void* out, void* final_state, void* workspace,
                     void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
                     int sdt, size_t workspace_bytes, const kda_strides_t& sd,
                     void* checkpoints = nullptr, int32_t ck_interval = 0,
                     int64_t ck_capacity = 0, const int32_t* sp_idx = nullptr,
                     const int32_t* sp_acc = nullptr, int32_t sp_stride = 0, int64_t sp_slots = 0,
                     int32_t* fixed_status = nullptr, bool fixed_scratch = false) {
  // ---- checks (no HIP call before they pass) --------------------------------
  if (num_tokens < 0 || num_tokens > INT32_MAX) return KDA_ERR_INVALID_ARG;  // int32 offsets
  // per-token tensors may be empty (and NULL) only when there are no tokens
  if (num_tokens > 0 && (!q || !k || !v || !g || !beta_logits || !out)) return KDA_ERR_INVALID_ARG;
  if (!A_log || !dt_bias || !cu_seqlens || !final_state) return KDA_ERR_INVALID_ARG;
  if (heads <= 0 || heads > 65536 || num_seqs <= 0) return KDA_ERR_INVALID_ARG;
  // the kernels address token rows with 32-bit byte offsets, also rows up to
  // 256 past a sequence's end (range-checked reads that return zeros), with
  // 8- and 16-byte accesses
  const int64_t T = num_tokens, H = heads;
  if (!rows_ok(sd.q_token, sd.q_head, T, H, KDA_HEAD_DIM, 8) ||
      !rows_ok(sd.k_token, sd.k_head, T, H, KDA_HEAD_DIM, 8) ||
      !rows_ok(sd.v_token, sd.v_head, T, H, KDA_HEAD_DIM, 8) ||
      !rows_ok(sd.g_token, sd.g_head, T, H, KDA_HEAD_DIM, 8) ||
      !rows_ok(sd.out_token, sd.out_head, T, H, KDA_HEAD_DIM, 8) ||
      !rows_ok(sd.beta_token, sd.beta_head, T, H, 1, 1))
    return KDA_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, g, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(beta_logits) % 2) return KDA_ERR_INVALID_ARG;
  // grid size: one workgroup per (sequence, head, value slice), up to 8 slices
  if (int64_t(num_seqs) * heads * 8 > INT32_MAX) return KDA_ERR_INVALID_ARG;
  if (sdt != KDA_STATE_FP32 && sdt != KDA_STATE_BF16) return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(lower_bound) || !std::isfinite(scale)) return KDA_ERR_INVALID_ARG;
  if (lower_bound > 0.f || lower_bound < KDA_LOWER_BOUND_MIN) return KDA_ERR_UNSUPPORTED;
  if (checkpoints) {
    if (ck_interval <= 0 || ck_interval % 16) return KDA_ERR_INVALID_ARG;
    if (ck_capacity < num_tokens / ck_interval) return KDA_ERR_INVALID_ARG;
  }
  if (sp_idx) {
    if (!sp_acc || sp_stride <= 0 || sp_slots <= 0) return KDA_ERR_INVALID_ARG;
    // slot offsets: sp_slots * heads * 128 * 128 elements
    if (sp_slots > (INT64_MAX / 4) / (int64_t(heads) * KDA_HEAD_DIM * KDA_HEAD_DIM))
      return KDA_ERR_INVALID_ARG;
  }
  if (fixed_scratch) {
    // no workspace: the status word is the caller's, the order table the
    // library's static scratch
    if (!fixed_status) return KDA_ERR_INVALID_ARG;
    if (num_seqs > kNoAllocMaxSeqs) return KDA_ERR_INVALID_ARG;
  } else {
    // the segment area is optional: without it the call takes the plain schedule
    const size_t need = base_workspace_bytes(num_seqs);
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace) return KDA_ERR_INVALID_ARG;
  }

  // ---- plan --------------------------------------------------------------------
  int cus = 0;
  if (hipError_t e = device_cu_count(&cus); e != hipSuccess) return hip_failure(e, "device query");
  const int forced = g_vsplit_override.load(std::memory_order_relaxed);
  const int s = forced > 0 ? forced : plan_vsplit(heads, num_seqs, cus);

  kda::Params p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g);
  p.beta = static_cast<const uint16_t*>(beta_logits);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.s0 = initial_state;
  p.sT = final_state;
  p.out = static_cast<uint16_t*>(out);
  p.cu = cu_seqlens;
  if (fixed_scratch) {
    p.errword = fixed_status;
    if (hipError_t e = scratch_address(&p.order); e != hipSuccess)
      return hip_failure(e, "scratch address query");
  } else {
    p.errword = static_cast<int32_t*>(workspace);
    p.order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kAlign);
  }
  p.lower_bound = lower_bound;
  p.scale = scale;
  p.ts_q = int(sd.q_token), p.hs_q = int(sd.q_head);
  p.ts_k = int(sd.k_token), p.hs_k = int(sd.k_head);
  p.ts_v = int(sd.v_token), p.hs_v = int(sd.v_head);
  p.ts_g = int(sd.g_token), p.hs_g = int(sd.g_head);
  p.ts_b = int(sd.beta_token), p.hs_b = int(sd.beta_head);
  p.ts_o = int(sd.out_token), p.hs_o = int(sd.out_head);
  p.T = int(num_tokens);
  p.H = heads;
  p.N = num_seqs;
  p.vsplit = s;
  p.state_bf16 = sdt == KDA_STATE_BF16;
  p.ck = checkpoints;
  p.ck_int = ck_interval;
  p.ck_cap = ck_capacity;
  p.sp_idx = sp_idx;
  p.sp_acc = sp_acc;
  p.sp_stride = sp_stride;
  p.sp_slots = sp_slots;

  hipStream_t st = static_cast<hipStream_t>(stream);
  // kernel families: 4 the pipelined 16-token kernel (default for
  // lower_bound >= kPipeLowerBoundMin), 5 the pipelined 32-token kernel (its
  // two 16-token halves keep their own decay references, so it serves
  // lower_bound down to KDA_LOWER_BOUND_MIN), 3 the decode kernel for
  // decode-sized calls (at most kDecodeTokensPerSeq tokens per sequence on
  // average: it streams each state once with 16-byte accesses and the chunked
  // machinery does not pay off), 1 and 2 on request (test hook)
  const int override = g_kernel_override.load(std::memory_order_relaxed);
  int kernel = override;
  if (kernel == 0)
    kernel = (!checkpoints && num_tokens <= kda::kDecodeTokensPerSeq * int64_t(num_seqs)) ? 3 : 4;
  // a speculative-decode step runs on the token-serial kernels, which store
  // the state after every token
  if (sp_idx) {
    if (override != 0 && override != 2 && override != 3) return KDA_ERR_UNSUPPORTED;
    kernel = override == 2 ? 2 : 3;
  }
  // the 16-token kernel takes lower_bound >= -5 and slices of <= 64 value
  // columns: below that bound the 32-token kernel, an unsplit launch (test
  // hook) the 64-token kernel.  Both pipelined kernels split the value
  // dimension at least in two when the rule says unsplit (a 128-column slice
  // holds more state than their waves' registers: measured slower; the
  // two-workgroup form below is the unsplit one).  Kernel 6 (the two-workgroup
  // form on request) falls back to the 16-token kernel where it cannot run.
  const bool want_duo = kernel == 6;
  if (kernel == 6) kernel = 4;
  if (kernel == 4 && lower_bound < kda::kPipeLowerBoundMin) kernel = 5;
  if ((kernel == 4 || kernel == 5) && p.vsplit == 1 && forced == 0) p.vsplit = 2;
  if (kernel == 4 && p.vsplit == 1) kernel = 1;
  if (checkpoints && kernel != 4 && kernel != 5) return KDA_ERR_UNSUPPORTED;

  // segment-parallel schedule: summaries, combine, rerun (kda_segment.hip)
  if (kernel == 4 && !want_duo && !checkpoints && !sp_idx && !fixed_scratch &&
      reinterpret_cast<uintptr_t>(workspace) % 16 == 0) {
    const int L = plan_segment_len(num_tokens, heads, num_seqs,
                                   g_segment_override.load(std::memory_order_relaxed));
    const SegLayout lay = seg_layout();
    const size_t off = base_workspace_bytes(num_seqs);
    if (L > 0 && workspace_bytes >= off + lay.bytes) {
      char* w = static_cast<char*>(workspace) + off;
      kda::SegParams sp{};
      sp.cu = cu_seqlens;
      sp.N = num_seqs;
      sp.T = int(num_tokens);
      sp.H = heads;
      sp.L = L;
      sp.M = num_seqs + int(num_tokens / L);
      sp.table = reinterpret_cast<int32_t*>(w + lay.table);
      sp.first = reinterpret_cast<int32_t*>(w + lay.first);
      sp.count = reinterpret_cast<int32_t*>(w + lay.count);
      sp.s0 = initial_state;
      sp.s0_bf16 = sdt == KDA_STATE_BF16;
      sp.summ = reinterpret_cast<const float*>(w + lay.summ);
      sp.starts = reinterpret_cast<float*>(w + lay.starts);
      if (hipError_t e = kda::launch_seg_plan(sp, st); e != hipSuccess)
        return hip_failure(e, "segment plan launch");
      kda::Params pa = p;  // summaries: [local state | transition], 4 slices of 64
      pa.seg = sp.table;
      pa.seg_mode = 1;
      pa.N = sp.M;
      pa.vsplit = 4;
      pa.order = nullptr;
      pa.s0 = nullptr;
      pa.sT = const_cast<float*>(sp.summ);
      pa.state_bf16 = 0;
      if (hipError_t e = kda::launch_pipe(pa, st); e != hipSuccess)
        return hip_failure(e, "segment summary launch");
      if (hipError_t e = kda::launch_seg_combine(sp, st); e != hipSuccess)
        return hip_failure(e, "segment combine launch");
      kda::Params pc = p;  // rerun of every segment from its entering state
      pc.seg = sp.table;
      pc.seg_mode = 2;
      pc.N = sp.M;
      pc.vsplit = forced > 0 ? forced : std::max(2, plan_vsplit(heads, sp.M, cus));
      pc.order = nullptr;
      pc.s0 = sp.starts;
      if (hipError_t e = kda::launch_pipe(pc, st); e != hipSuccess)
        return hip_failure(e, "segment rerun launch");
      return KDA_OK;
    }
  }

  // two-workgroup forward: automatic in its range of item counts, or on
  // request (kernel 6, any count that fits; else the plain kernel)
  if (kernel == 4 && !checkpoints && !sp_idx && !fixed_scratch &&
      reinterpret_cast<uintptr_t>(workspace) % 16 == 0 && forced == 0) {
    const SegLayout lay = seg_layout();
    const size_t off = base_workspace_bytes(num_seqs);
    if (workspace_bytes >= off + lay.bytes && duo_rule(num_tokens, heads, num_seqs, cus, want_duo)) {
      char* w = static_cast<char*>(workspace) + off;
      p.duo_ring = w + lay.summ;
      p.duo_flags = reinterpret_cast<uint64_t*>(w + lay.duo_flags);
      uint32_t nonce = 0;
      while (nonce == 0) nonce = g_duo_nonce.fetch_add(0x9e3779b9u, std::memory_order_relaxed);
      p.duo_nonce = nonce;
      p.order = nullptr;
      if (hipError_t e = kda::launch_duo(p, st); e != hipSuccess)
        return hip_failure(e, "two-workgroup kernel launch");
      return KDA_OK;
    }
  }

  // the sequence order table (longest first): the pipelined kernels rank a
  // few sequences themselves, the decode path takes them in index order, the
  // others read the table
  if (((kernel == 4 || kernel == 5) && num_seqs <= kda::kInlineRankMax) || kernel == 3) {
    p.order = nullptr;
  } else if (hipError_t e = kda::launch_plan(p, st); e != hipSuccess) {
    return hip_failure(e, "plan launch");
  }
  if (kernel == 2 || kernel == 3) {
    if (hipError_t e = kda::launch_recurrent(p, st, kernel == 3); e != hipSuccess)
      return hip_failure(e, "token-serial kernel launch");
  } else if (kernel == 1) {
    if (hipError_t e = kda::launch_chunk(p, st); e != hipSuccess)
      return hip_failure(e, "64-token chunk kernel launch");
  } else if (kernel == 4) {
    if (hipError_t e = kda::launch_pipe(p, st); e != hipSuccess)
      return hip_failure(e, "pipelined 16-token kernel launch");
  } else {
    if (hipError_t e = kda::launch_fwd32(p, st); e != hipSuccess)
      return hip_failure(e, "pipelined 32-token kernel launch");
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_prefill_fwd(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta_logits, const float* A_log,
                                   const float* dt_bias, float lower_bound, float scale,
                                   const void* initial_state, const int32_t* cu_seqlens, void* out,
                                   void* final_state, void* workspace, void* stream,
                                   int64_t num_tokens, int32_t heads, int32_t num_seqs,
                                   kda_state_dtype_t state_dtype, size_t workspace_bytes) {
  const int64_t row = int64_t(heads) * KDA_HEAD_DIM;
  const kda_strides_t dense{row, KDA_HEAD_DIM, row, KDA_HEAD_DIM, row,   KDA_HEAD_DIM,
                            row, KDA_HEAD_DIM, heads, 1,          row, KDA_HEAD_DIM};
  return forward(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale, initial_state,
                 cu_seqlens, out, final_state, workspace, stream, num_tokens, heads, num_seqs,
                 enum_value(state_dtype), workspace_bytes, dense);
}

size_t kda_gate_proj_workspace_size(int32_t num_tokens, int32_t hidden_dim, int32_t n_ab) {
  if (num_tokens < 0 || hidden_dim <= 0 || n_ab <= 0) return 0;
  return kda::proj_workspace_bytes(num_tokens, hidden_dim, n_ab);
}

kda_status_t kda_gate_proj(const void* hidden, const void* w_ab, const void* w_b, void* p_ab,
                           void* g, void* workspace, size_t workspace_bytes, void* stream,
                           int32_t num_tokens, int32_t hidden_dim, int32_t n_ab, int32_t n_b) {
  // ---- checks (no HIP call before they pass) --------------------------------
  if (num_tokens < 0 || num_tokens > (1 << 16)) return KDA_ERR_INVALID_ARG;
  if (hidden_dim <= 0 || hidden_dim % 8 || hidden_dim > (1 << 24)) return KDA_ERR_INVALID_ARG;
  if (n_ab < kda::kProjRank || n_ab % 8 || n_ab > 4096) return KDA_ERR_INVALID_ARG;
  if (n_b <= 0 || n_b % 16 || n_b > (1 << 20)) return KDA_ERR_INVALID_ARG;
  if (!w_ab || !w_b) return KDA_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!hidden || !p_ab || !g)) return KDA_ERR_INVALID_ARG;
  for (const void* ptr : {hidden, w_ab, w_b, static_cast<const void*>(p_ab)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(g) % 2) return KDA_ERR_INVALID_ARG;
  const size_t need = kda_gate_proj_workspace_size(num_tokens, hidden_dim, n_ab);
  if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if (num_tokens == 0) return KDA_OK;  // (needs no workspace)
  if (!workspace) return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return KDA_ERR_INVALID_ARG;

  kda::ProjParams pp{};
  pp.hidden = static_cast<const uint16_t*>(hidden);
  pp.w_ab = static_cast<const uint16_t*>(w_ab);
  pp.w_b = static_cast<const uint16_t*>(w_b);
  pp.p_ab = static_cast<uint16_t*>(p_ab);
  pp.g = static_cast<uint16_t*>(g);
  pp.partials = static_cast<float*>(workspace);
  pp.M = num_tokens;
  pp.K = hidden_dim;
  pp.n_ab = n_ab;
  pp.n_b = n_b;
  if (hipError_t e = kda::launch_proj(pp, static_cast<hipStream_t>(stream)); e != hipSuccess)
    return hip_failure(e, "projection launch");
  return KDA_OK;
}

kda_status_t kda_chunk_prefill_fwd_noalloc(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    int32_t* status, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype) {
  const int64_t row = int64_t(heads) * KDA_HEAD_DIM;
  const kda_strides_t dense{row, KDA_HEAD_DIM, row, KDA_HEAD_DIM, row,   KDA_HEAD_DIM,
                            row, KDA_HEAD_DIM, heads, 1,          row, KDA_HEAD_DIM};
  return forward(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale, initial_state,
                 cu_seqlens, out, final_state, nullptr, stream, num_tokens, heads, num_seqs,
                 enum_value(state_dtype), 0, dense, nullptr, 0, 0, nullptr, nullptr, 0, 0, status,
                 true);
}

kda_status_t kda_spec_decode_step(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale, void* state_pool,
    int64_t num_slots, const int32_t* cu_seqlens, const int32_t* state_indices,
    int32_t indices_stride, const int32_t* num_accepted_tokens, void* out, void* workspace,
    void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes) {
  if (!state_pool || !state_indices) return KDA_ERR_INVALID_ARG;
  const int64_t row = int64_t(heads) * KDA_HEAD_DIM;
  const kda_strides_t dense{row, KDA_HEAD_DIM, row, KDA_HEAD_DIM, row,   KDA_HEAD_DIM,
                            row, KDA_HEAD_DIM, heads, 1,          row, KDA_HEAD_DIM};
  return forward(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale, state_pool,
                 cu_seqlens, out, state_pool, workspace, stream, num_tokens, heads, num_seqs,
                 enum_value(state_dtype), workspace_bytes, dense, nullptr, 0, 0, state_indices,
                 num_accepted_tokens, indices_stride, num_slots);
}

kda_status_t kda_chunk_prefill_fwd_checkpoints(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    void* workspace, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes, const kda_strides_t* strides,
    void* checkpoints, int32_t checkpoint_interval, int64_t checkpoint_capacity) {
  if (!checkpoints) return KDA_ERR_INVALID_ARG;
  const int64_t row = int64_t(heads) * KDA_HEAD_DIM;
  const kda_strides_t dense{row, KDA_HEAD_DIM, row, KDA_HEAD_DIM, row,   KDA_HEAD_DIM,
                            row, KDA_HEAD_DIM, heads, 1,          row, KDA_HEAD_DIM};
  return forward(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale, initial_state,
                 cu_seqlens, out, final_state, workspace, stream, num_tokens, heads, num_seqs,
                 enum_value(state_dtype), workspace_bytes, strides ? *strides : dense, checkpoints,
                 checkpoint_interval, checkpoint_capacity);
}

kda_status_t kda_chunk_prefill_fwd_strided(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    void* workspace, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes, const kda_strides_t* strides) {
  if (!strides) return KDA_ERR_INVALID_ARG;
  return forward(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale, initial_state,
                 cu_seqlens, out, final_state, workspace, stream, num_tokens, heads, num_seqs,
                 enum_value(state_dtype), workspace_bytes, *strides);
}

}  // extern "C"
