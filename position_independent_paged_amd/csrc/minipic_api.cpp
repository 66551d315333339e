// Host side of libminipic.so: argument validation, launch planning and
// dispatch. Every check here reads host values only and runs before the first
// HIP call, so a rejected call never touches the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/minipic.h"
#include "../../include/minipic_desc.h"
#include "common.h"

namespace minipic {
hipError_t launch_plan(const PlanParams& p, int bq, hipStream_t s);
hipError_t launch_attn_bf16(const AttnParams& p, int D, int G, bool rope, int grid, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int D, int G, bool rope, int grid, hipStream_t s);
int attn_bf16_blocks_per_cu(int D, int G, bool rope);
int attn_bf16_rows();
int attn_bf16_threads();
int attn_f32_blocks_per_cu(int D, int G, bool rope);
hipError_t launch_write_kv(const void* k, const void* v, const int64_t* slots, int64_t n, int hkv, int D,
                           void* kc, void* vc, int64_t num_blocks, int dtype, hipStream_t s);
hipError_t launch_rope_table(float* cs, int max_pos, int d, double base, hipStream_t s);
hipError_t launch_merge(const AttnParams& p, int D, int dtype, int rows, int G, int max_groups, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeParams& p, int D, int G, bool rope, hipStream_t s);
hipError_t launch_decode_merge(const DecodeParams& p, int D, int G, hipStream_t s);
}  // namespace minipic

using namespace minipic;

// Workspace of minipic_prefill_attn_static: device memory the library owns,
// one copy on every GPU that runs that entry point, held until the process
// ends. On the host this name stands for a host-side stand-in, not a device
// address; host code takes each device's address from hipGetSymbolAddress
// (static_workspace below) and never uses the name itself.
static __device__ __align__(256) unsigned char scratch[MINIPIC_STATIC_WORKSPACE_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MINIPIC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Host-side plan: sizes from host scalars only.
struct Plan {
  int rows, bq, nqt, threads, min_chunk, slots, max_groups;
  int64_t tiles, max_items;
  size_t off_tiles, off_toks, off_blist, off_items, off_groups, off_ml, off_o, bytes;
};

constexpr size_t kAlign = 256;
constexpr int kSlotCap = 512;   // partial-result slots: room for two pieces per CU of a 256-CU GPU
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_batch(const minipic_batch* b, int dtype) {
  if (!b) return fail(MINIPIC_ERR_INVALID_ARG, "batch is NULL");
  if (dtype != MINIPIC_F32 && dtype != MINIPIC_BF16)
    return fail(MINIPIC_ERR_UNSUPPORTED, "dtype %d is not MINIPIC_F32 or MINIPIC_BF16", dtype);
  if (b->num_reqs < 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_reqs < 0");
  if (b->num_q_heads <= 0 || b->num_kv_heads <= 0)
    return fail(MINIPIC_ERR_INVALID_ARG, "head counts must be positive");
  if (b->num_kv_heads > 255)   // work items pack the KV head into 8 bits
    return fail(MINIPIC_ERR_UNSUPPORTED, "num_kv_heads must be at most 255 (got %d)", b->num_kv_heads);
  if (b->num_q_heads % b->num_kv_heads != 0)
    return fail(MINIPIC_ERR_UNSUPPORTED, "num_q_heads %% num_kv_heads != 0");
  if (!supported_group(b->num_q_heads / b->num_kv_heads))
    return fail(MINIPIC_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)",
                b->num_q_heads / b->num_kv_heads);
  if (!supported_dim(b->head_dim)) return fail(MINIPIC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (b->block_size != kBlock) return fail(MINIPIC_ERR_UNSUPPORTED, "block_size must be 16");
  if (b->max_blocks_per_req <= 0) return fail(MINIPIC_ERR_INVALID_ARG, "max_blocks_per_req must be > 0");
  if (b->total_q < 0 || b->max_q_len < 0 || b->max_ctx_len < 0)
    return fail(MINIPIC_ERR_INVALID_ARG, "negative size in batch");
  if ((int64_t)b->max_ctx_len > (int64_t)b->max_blocks_per_req * kBlock)
    return fail(MINIPIC_ERR_INVALID_ARG, "max_ctx_len exceeds max_blocks_per_req * block_size");
  if (b->total_q > 0 && b->max_q_len == 0) return fail(MINIPIC_ERR_INVALID_ARG, "max_q_len is 0 but total_q > 0");
  if (b->num_reqs > 0 && b->total_q > 0) {
    if (!b->q_indptr || !b->q_ctx_idx || !b->ctx_len || !b->block_table || !b->logical_pos || !b->span_id ||
        !b->blk_flags)
      return fail(MINIPIC_ERR_INVALID_ARG, "a batch array pointer is NULL");
  }
  if (b->total_q > (int64_t)INT32_MAX) return fail(MINIPIC_ERR_INVALID_ARG, "total_q too large");
  if ((uintptr_t)b->logical_pos % 16) return fail(MINIPIC_ERR_INVALID_ARG, "logical_pos must be 16-byte aligned");
  return MINIPIC_OK;
}

// The kernels address the cos/sin table through a buffer range of 32-bit size.
int check_table(const float* cos_sin, int32_t max_pos, int head_dim) {
  if (!cos_sin) return fail(MINIPIC_ERR_INVALID_ARG, "cos_sin is NULL");
  if (max_pos <= 0) return fail(MINIPIC_ERR_INVALID_ARG, "max_pos must be > 0");
  if ((int64_t)max_pos * head_dim * (int64_t)sizeof(float) > (int64_t)INT32_MAX)
    return fail(MINIPIC_ERR_INVALID_ARG, "cos/sin table of %d rows x %d floats exceeds 2^31 bytes", max_pos, head_dim);
  return MINIPIC_OK;
}

// Optional kernel timing (minipic_set_kernel_timing): events recorded on the
// call's stream around the three launches of each call of this thread, one
// set of four per call for up to kTimedCalls calls since timing was switched
// on (later calls reuse the sets in turn). Events are created on first use
// and kept until the process ends.
constexpr int kTimedCalls = 4096;
struct KernelTimer {
  bool on = false;
  bool valid = false;      // the latest call was timed completely
  int64_t calls = 0;       // calls begun since timing was switched on
  std::vector<hipEvent_t> ev;   // [kTimedCalls][4]
};
thread_local KernelTimer g_timer;

hipError_t timer_mark(int i, hipStream_t s) {
  if (!g_timer.on) return hipSuccess;
  if (i == 0) ++g_timer.calls;
  if (g_timer.ev.empty()) g_timer.ev.assign((size_t)kTimedCalls * 4, nullptr);
  hipEvent_t& e = g_timer.ev[(size_t)((g_timer.calls - 1) % kTimedCalls) * 4 + i];
  if (!e) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return r;
  }
  return hipEventRecord(e, s);
}

// Decode plan (host scalars only): key splits per (request, KV head) so that
// about kDecodeWaves waves (one round at two waves per SIMD on 256 CUs) cover
// the batch, every split at least two blocks, at most kDecodeMaxSplits splits.
constexpr int64_t kDecodeWaves = 2048;
struct DecodePlan {
  int split_blocks, nsplit;
  size_t off_ml, off_o, bytes;
};

void make_decode_plan(const minipic_batch* b, DecodePlan* p) {
  const int64_t MB = b->max_blocks_per_req;
  const int64_t per = (int64_t)b->num_reqs * b->num_kv_heads * MB;
  int64_t sb = (per + kDecodeWaves - 1) / kDecodeWaves;
  if (sb < 2) sb = 2;
  if ((MB + sb - 1) / sb > kDecodeMaxSplits) sb = (MB + kDecodeMaxSplits - 1) / kDecodeMaxSplits;
  p->split_blocks = (int)sb;
  p->nsplit = (int)((MB + sb - 1) / sb);
  const int64_t parts = (int64_t)b->num_reqs * b->num_q_heads * p->nsplit;   // (request, KV head, split, head in group)
  size_t off = kAlign;   // header: the error word
  p->off_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)parts);
  p->off_o = off;
  off = align_up(off + sizeof(float) * (size_t)parts * b->head_dim);
  p->bytes = off;
}

int check_decode(const minipic_batch* b, int dtype) {
  int st = check_batch(b, dtype);
  if (st) return st;
  if (dtype != MINIPIC_BF16) return fail(MINIPIC_ERR_UNSUPPORTED, "decode attention supports MINIPIC_BF16 only");
  if (b->total_q != b->num_reqs)
    return fail(MINIPIC_ERR_INVALID_ARG, "decode takes one query row per request (total_q %lld, num_reqs %d)",
                (long long)b->total_q, b->num_reqs);
  return MINIPIC_OK;
}

int run_decode(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
               const minipic_batch* b, const float* cos_sin, int32_t max_pos, float softmax_scale, void* out,
               void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype, void* stream, bool rope) {
  int st = check_decode(b, dtype);
  if (st) return st;
  if (flags) return fail(MINIPIC_ERR_INVALID_ARG, "decode takes no flags (q arrives rotated), got 0x%x", flags);
  if (num_blocks < 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_blocks < 0");
  if (rope) {
    st = check_table(cos_sin, max_pos, b->head_dim);
    if (st) return st;
  }
  if (b->num_reqs == 0) return MINIPIC_OK;
  if (!q || !out) return fail(MINIPIC_ERR_INVALID_ARG, "q or out is NULL");
  if (!k_cache || !v_cache) return fail(MINIPIC_ERR_INVALID_ARG, "k_cache or v_cache is NULL");
  if (num_blocks == 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_blocks is 0");
  if (!(softmax_scale == softmax_scale) || std::isinf(softmax_scale))
    return fail(MINIPIC_ERR_INVALID_ARG, "softmax_scale is not finite");
  DecodePlan pl;
  make_decode_plan(b, &pl);
  if (!workspace) return fail(MINIPIC_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(MINIPIC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(MINIPIC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
  if ((int64_t)b->num_reqs * b->num_kv_heads * pl.nsplit > (int64_t)INT32_MAX / 2)
    return fail(MINIPIC_ERR_INVALID_ARG, "batch too large for one launch");
  char* ws = (char*)workspace;
  DecodeParams P{};
  P.q = q;
  P.k_cache = k_cache;
  P.v_cache = v_cache;
  P.out = out;
  P.cos_sin = cos_sin;
  P.q_ctx_idx = b->q_ctx_idx;
  P.ctx_len = b->ctx_len;
  P.block_table = b->block_table;
  P.logical_pos = b->logical_pos;
  P.span_id = b->span_id;
  P.blk_flags = b->blk_flags;
  P.err = (uint32_t*)ws;
  P.part_ml = (float2*)(ws + pl.off_ml);
  P.part_o = (float*)(ws + pl.off_o);
  P.num_blocks = num_blocks;
  P.num_reqs = b->num_reqs;
  P.hq = b->num_q_heads;
  P.hkv = b->num_kv_heads;
  P.max_blocks = b->max_blocks_per_req;
  P.max_pos = rope ? max_pos : 1;
  P.nsplit = pl.nsplit;
  P.split_blocks = pl.split_blocks;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)b->head_dim);
  P.scale_log2 = scale * 1.4426950408889634f;
  const int G = b->num_q_heads / b->num_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  g_timer.valid = false;
  hipError_t e = timer_mark(0, s);
  if (e == hipSuccess) e = timer_mark(1, s);
  if (e == hipSuccess) e = launch_decode_bf16(P, b->head_dim, G, rope, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = timer_mark(2, s);
  if (e == hipSuccess) e = launch_decode_merge(P, b->head_dim, G, s);
  if (e == hipSuccess) e = timer_mark(3, s);
  if (e != hipSuccess) return hip_fail(e, "decode merge launch");
  g_timer.valid = g_timer.on;
  return MINIPIC_OK;
}

// Device address of `scratch` on the current device: hipGetSymbolAddress on
// the first call on each device (with that device current, return code
// checked), the kept address after that.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int static_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MINIPIC_ERR_UNSUPPORTED, "device %d: the static workspace serves devices 0..%d", dev, kMaxDevices - 1);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p || (uintptr_t)p % kAlign) return fail(MINIPIC_ERR_HIP, "static workspace at %p is not 256-byte aligned", p);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MINIPIC_OK;
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

void make_plan(const minipic_batch* b, int dtype, Plan* p) {
  const int G = b->num_q_heads / b->num_kv_heads;
  if (dtype == MINIPIC_BF16) {
    p->rows = attn_bf16_rows();
    p->threads = attn_bf16_threads();
  } else {
    p->rows = 64;
    p->threads = 256;
  }
  p->bq = p->rows / G;
  p->nqt = b->max_q_len > 0 ? (b->max_q_len + p->bq - 1) / p->bq : 0;
  p->tiles = (int64_t)b->num_reqs * p->nqt;
  p->min_chunk = env_int("MINIPIC_MIN_CHUNK", 16);
  if (p->min_chunk < 1) p->min_chunk = 1;
  const int64_t hkv = b->num_kv_heads;
  int64_t slots = p->tiles * hkv * kMaxSplits;
  // MINIPIC_SLOT_CAP lowers the cap (tuning and tests of the planner's
  // piece-doubling path); it never raises it past the workspace plan
  int cap = env_int("MINIPIC_SLOT_CAP", kSlotCap);
  if (cap < 2 || cap > kSlotCap) cap = kSlotCap;
  if (slots > cap) slots = cap;
  p->slots = (int)slots;
  p->max_items = p->tiles * hkv + p->slots;
  size_t off = kAlign;  // WsHeader
  p->off_tiles = off;
  off = align_up(off + sizeof(TileDesc) * (size_t)p->tiles);
  p->off_toks = off;
  off = align_up(off + sizeof(TokDesc) * (size_t)p->tiles * p->bq);
  p->off_blist = off;
  off = align_up(off + sizeof(BlkDesc) * (size_t)p->tiles * b->max_blocks_per_req);
  p->off_items = off;
  off = align_up(off + sizeof(Item) * (size_t)p->max_items);
  p->max_groups = p->slots / 2 > 0 ? p->slots / 2 : 1;  // a split group holds >= 2 pieces
  p->off_groups = off;
  off = align_up(off + sizeof(Group) * (size_t)p->max_groups);
  p->off_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)p->slots * p->rows);
  p->off_o = off;
  off = align_up(off + sizeof(float) * (size_t)p->slots * p->rows * b->head_dim);
  p->bytes = off;
}

// Persistent grid of the attention kernel on the current device: CUs times
// resident work-groups per CU, cached per (device, kernel configuration).
int persistent_grid(int dtype, int D, int G, bool rope, int* grid) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  static thread_local int cache[64][2][2][4][2];
  const int di = dtype == MINIPIC_BF16 ? 1 : 0;
  const int Di = D == 128 ? 1 : 0;
  const int Gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  int* c = dev < 64 ? &cache[dev][di][Di][Gi][rope ? 1 : 0] : nullptr;
  if (c && *c > 0) {
    *grid = *c;
    return 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
  const int per_cu = dtype == MINIPIC_BF16 ? attn_bf16_blocks_per_cu(D, G, rope) : attn_f32_blocks_per_cu(D, G, rope);
  int g = cus * per_cu;
  const int over = env_int("MINIPIC_GRID", 0);
  if (over > 0) g = over;
  if (c) *c = g;
  *grid = g;
  return 0;
}

// Key of a plan's configuration: FNV-1a over everything the planning kernels
// read or size their output by (the batch's scalars and array addresses,
// num_blocks, the table rows and flags, the dtype, the kernel variant and the
// launch size). Never 0, so a zeroed workspace holds no plan.
uint64_t plan_key(const minipic_batch* b, int32_t dtype, bool rope, uint32_t flags, int32_t max_pos_used,
                  int64_t num_blocks, int grid) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix((uint64_t)(uint32_t)dtype);
  mix(rope ? 1u : 0u);
  mix(flags);
  mix((uint64_t)(uint32_t)max_pos_used);
  mix((uint64_t)num_blocks);
  mix((uint64_t)(uint32_t)grid);
  mix((uint64_t)(uint32_t)b->num_reqs);
  mix((uint64_t)(uint32_t)b->num_q_heads);
  mix((uint64_t)(uint32_t)b->num_kv_heads);
  mix((uint64_t)(uint32_t)b->head_dim);
  mix((uint64_t)(uint32_t)b->block_size);
  mix((uint64_t)(uint32_t)b->max_blocks_per_req);
  mix((uint64_t)b->total_q);
  mix((uint64_t)(uint32_t)b->max_q_len);
  mix((uint64_t)(uintptr_t)b->q_indptr);
  mix((uint64_t)(uintptr_t)b->q_ctx_idx);
  mix((uint64_t)(uintptr_t)b->ctx_len);
  mix((uint64_t)(uintptr_t)b->block_table);
  mix((uint64_t)(uintptr_t)b->logical_pos);
  mix((uint64_t)(uintptr_t)b->span_id);
  mix((uint64_t)(uintptr_t)b->blk_flags);
  return h == 0 ? 1 : h;
}

// What a prefill entry point launches: the planning kernels, the attention
// and merge kernels, or both.
enum class Mode { kPlanAndRun, kPlan, kRun };

int run_attention(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                  const minipic_batch* b, const float* cos_sin, int32_t max_pos, float softmax_scale,
                  void* out, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype,
                  void* stream, bool rope, bool static_ws = false, uint32_t* err_word = nullptr,
                  Mode mode = Mode::kPlanAndRun) {
  const bool do_plan = mode != Mode::kRun, do_run = mode != Mode::kPlan;
  int st = check_batch(b, dtype);
  if (st) return st;
  if (flags & ~(uint32_t)MINIPIC_FLAG_ROTATE_Q) return fail(MINIPIC_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (num_blocks < 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_blocks < 0");
  const bool need_table = rope || (flags & MINIPIC_FLAG_ROTATE_Q);
  if (need_table) {
    st = check_table(cos_sin, max_pos, b->head_dim);
    if (st) return st;
  }
  if (b->num_reqs == 0 || b->total_q == 0) return MINIPIC_OK;
  if (do_run) {
    if (!q || !out) return fail(MINIPIC_ERR_INVALID_ARG, "q or out is NULL");
    if (!k_cache || !v_cache) return fail(MINIPIC_ERR_INVALID_ARG, "k_cache or v_cache is NULL");
  }
  if (num_blocks == 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_blocks is 0");
  if (do_run && (!(softmax_scale == softmax_scale) || std::isinf(softmax_scale)))
    return fail(MINIPIC_ERR_INVALID_ARG, "softmax_scale is not finite");
  Plan pl;
  make_plan(b, dtype, &pl);
  if (static_ws) {
    if ((uintptr_t)err_word % alignof(uint32_t)) return fail(MINIPIC_ERR_INVALID_ARG, "err_word must be 4-byte aligned");
    if (pl.bytes > (size_t)MINIPIC_STATIC_WORKSPACE_BYTES)
      return fail(MINIPIC_ERR_WORKSPACE, "batch needs %zu bytes of workspace; the static workspace holds %zu",
                  pl.bytes, (size_t)MINIPIC_STATIC_WORKSPACE_BYTES);
  } else {
    if (!workspace) return fail(MINIPIC_ERR_INVALID_ARG, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign) return fail(MINIPIC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < pl.bytes)
      return fail(MINIPIC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
  }
  if (pl.tiles > (int64_t)INT32_MAX / 2 || pl.max_items > (int64_t)INT32_MAX / 2)
    return fail(MINIPIC_ERR_INVALID_ARG, "batch too large for one launch");
  if (static_ws) {
    st = static_workspace(&workspace);
    if (st) return st;
  }
  const int G = b->num_q_heads / b->num_kv_heads;
  int grid = 0;
  if (persistent_grid(dtype, b->head_dim, G, rope, &grid) != 0)
    return fail(MINIPIC_ERR_HIP, "cannot query the current device");

  char* ws = (char*)workspace;
  PlanParams Q{};
  Q.q_indptr = b->q_indptr;
  Q.q_ctx_idx = b->q_ctx_idx;
  Q.ctx_len = b->ctx_len;
  Q.block_table = b->block_table;
  Q.span_id = b->span_id;
  Q.blk_flags = b->blk_flags;
  Q.hdr = (WsHeader*)ws;
  // the static workspace is shared by every call on the GPU: its error bits
  // go to the caller's word (or, without one, to a header word nobody reads)
  Q.err = static_ws && err_word ? err_word : &Q.hdr->err;
  Q.tiles = (TileDesc*)(ws + pl.off_tiles);
  Q.toks = (TokDesc*)(ws + pl.off_toks);
  Q.blist = (BlkDesc*)(ws + pl.off_blist);
  Q.items = (Item*)(ws + pl.off_items);
  Q.groups = (Group*)(ws + pl.off_groups);
  Q.num_blocks = num_blocks;
  Q.num_reqs = b->num_reqs;
  Q.nqt = pl.nqt;
  Q.num_tiles = (int)pl.tiles;
  Q.bq = pl.bq;
  Q.hkv = b->num_kv_heads;
  Q.max_blocks = b->max_blocks_per_req;
  Q.num_wg = grid;
  Q.max_slots = pl.slots;
  Q.max_items = (int)pl.max_items;
  Q.min_chunk = pl.min_chunk;
  Q.logical_pos = b->logical_pos;
  Q.max_pos = need_table ? max_pos : 1;
  Q.plan_key = plan_key(b, dtype, rope, flags, Q.max_pos, num_blocks, grid);

  AttnParams P{};
  P.q = q;
  P.k_cache = k_cache;
  P.v_cache = v_cache;
  P.out = out;
  P.cos_sin = cos_sin;
  P.logical_pos = b->logical_pos;
  P.hdr = Q.hdr;
  P.err = Q.err;
  P.tiles = Q.tiles;
  P.toks = Q.toks;
  P.blist = Q.blist;
  P.items = Q.items;
  P.groups = Q.groups;
  P.max_groups = pl.max_groups;
  P.part_ml = (float2*)(ws + pl.off_ml);
  P.part_o = (float*)(ws + pl.off_o);
  P.hq = b->num_q_heads;
  P.hkv = b->num_kv_heads;
  P.max_blocks = b->max_blocks_per_req;
  P.max_pos = need_table ? max_pos : 1;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)b->head_dim);
  P.scale_log2 = scale * 1.4426950408889634f;
  P.flags = flags;
  P.plan_key = Q.plan_key;
  P.num_wg = grid;
  hipStream_t s = (hipStream_t)stream;
  // calls on the static workspace record no timing events (creating them allocates)
  const bool timed = !static_ws;
  auto mark = [&](int i) { return timed ? timer_mark(i, s) : hipSuccess; };
  if (timed) g_timer.valid = false;
  if (mode == Mode::kPlan) {
    hipError_t e = launch_plan(Q, pl.bq, s);
    return e == hipSuccess ? MINIPIC_OK : hip_fail(e, "plan launch");
  }
  hipError_t e = mark(0);
  if (e == hipSuccess && do_plan) e = launch_plan(Q, pl.bq, s);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  e = mark(1);
  if (e == hipSuccess)
    e = dtype == MINIPIC_BF16 ? launch_attn_bf16(P, b->head_dim, G, rope, grid, s)
                              : launch_attn_f32(P, b->head_dim, G, rope, grid, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  e = mark(2);
  if (e == hipSuccess) e = launch_merge(P, b->head_dim, dtype, pl.rows, G, pl.max_groups, s);
  if (e == hipSuccess) e = mark(3);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  if (timed) g_timer.valid = g_timer.on;
  return MINIPIC_OK;
}

}  // namespace

namespace minipic_host {
int set_error(int code, const std::string& msg) { return fail(code, "%s", msg.c_str()); }
}  // namespace minipic_host

extern "C" {

const char* minipic_version(void) { return "minipic-mi355x 0.1.0 (gfx950)"; }

const char* minipic_status_string(int status) {
  switch (status) {
    case MINIPIC_OK: return "ok";
    case MINIPIC_ERR_INVALID_ARG: return "invalid argument";
    case MINIPIC_ERR_UNSUPPORTED: return "unsupported configuration";
    case MINIPIC_ERR_WORKSPACE: return "workspace too small";
    case MINIPIC_ERR_HIP: return "HIP error";
    case MINIPIC_ERR_CONTRACT: return "marker contract violated";
    case MINIPIC_ERR_CACHE_FULL: return "block cache full";
  }
  return "unknown status";
}

const char* minipic_last_error(void) { return g_last_error.c_str(); }

int minipic_rope_table(float* cos_sin, int32_t max_pos, int32_t head_dim, double base, void* stream) {
  if (!cos_sin) return fail(MINIPIC_ERR_INVALID_ARG, "cos_sin is NULL");
  if (max_pos <= 0) return fail(MINIPIC_ERR_INVALID_ARG, "max_pos must be > 0");
  if (head_dim <= 0 || head_dim % 2) return fail(MINIPIC_ERR_INVALID_ARG, "head_dim must be even and > 0");
  if (!(base > 0.0) || std::isinf(base)) return fail(MINIPIC_ERR_INVALID_ARG, "base must be finite and > 0");
  hipError_t e = launch_rope_table(cos_sin, max_pos, head_dim, base, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return MINIPIC_OK;
}

int minipic_write_kv(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, void* k_cache, void* v_cache,
                     int64_t num_blocks, int32_t dtype, void* stream) {
  if (dtype != MINIPIC_F32 && dtype != MINIPIC_BF16) return fail(MINIPIC_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (num_tokens < 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_kv_heads must be > 0");
  if (!supported_dim(head_dim)) return fail(MINIPIC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size != kBlock) return fail(MINIPIC_ERR_UNSUPPORTED, "block_size must be 16");
  if (num_blocks < 0) return fail(MINIPIC_ERR_INVALID_ARG, "num_blocks < 0");
  if (num_tokens == 0) return MINIPIC_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(MINIPIC_ERR_INVALID_ARG, "NULL pointer");
  if ((num_tokens + kBlock - 1) / kBlock > (int64_t)INT32_MAX) return fail(MINIPIC_ERR_INVALID_ARG, "too many tokens");
  hipError_t e = launch_write_kv(k, v, slot_mapping, num_tokens, num_kv_heads, head_dim, k_cache, v_cache,
                                 num_blocks, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "write_kv launch");
  return MINIPIC_OK;
}

int minipic_workspace_size(const minipic_batch* batch, int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(MINIPIC_ERR_INVALID_ARG, "bytes is NULL");
  int st = check_batch(batch, dtype);
  if (st) return st;
  Plan pl;
  make_plan(batch, dtype, &pl);
  *bytes = pl.bytes;
  return MINIPIC_OK;
}

int minipic_get_launch_info(const minipic_batch* batch, int32_t dtype, minipic_launch_info* info) {
  if (!info) return fail(MINIPIC_ERR_INVALID_ARG, "info is NULL");
  int st = check_batch(batch, dtype);
  if (st) return st;
  Plan pl;
  make_plan(batch, dtype, &pl);
  info->rows_per_tile = pl.rows;
  info->tokens_per_tile = pl.bq;
  info->num_q_tiles = pl.nqt;
  info->num_splits = kMaxSplits;
  info->split_blocks = pl.min_chunk;
  info->threads = pl.threads;
  int grid = 0, ndev = 0;
  info->num_workgroups = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0 &&
      persistent_grid(dtype, batch->head_dim, batch->num_q_heads / batch->num_kv_heads, true, &grid) == 0)
    info->num_workgroups = grid;
  info->num_tiles = pl.tiles;
  info->partial_slots = pl.slots;
  info->reserved = 0;
  return MINIPIC_OK;
}

int minipic_prefill_attn(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const minipic_batch* batch, const float* cos_sin, int32_t max_pos, float softmax_scale,
                         void* out, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype,
                         void* stream) {
  return run_attention(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, softmax_scale, out, workspace,
                       workspace_bytes, flags, dtype, stream, /*rope=*/true);
}

int minipic_prefill_attn_static(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                                const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                                float softmax_scale, void* out, uint32_t* err_word, uint32_t flags, int32_t dtype,
                                void* stream) {
  return run_attention(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, softmax_scale, out, nullptr, 0,
                       flags, dtype, stream, /*rope=*/true, /*static_ws=*/true, err_word);
}

int minipic_prefill_plan(int64_t num_blocks, const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                         void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype, void* stream) {
  return run_attention(nullptr, nullptr, nullptr, num_blocks, batch, cos_sin, max_pos, 0.f, nullptr, workspace,
                       workspace_bytes, flags, dtype, stream, /*rope=*/true, false, nullptr, Mode::kPlan);
}
int minipic_prefill_run(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                        const minipic_batch* batch, const float* cos_sin, int32_t max_pos, float softmax_scale,
                        void* out, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype,
                        void* stream) {
  return run_attention(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, softmax_scale, out, workspace,
                       workspace_bytes, flags, dtype, stream, /*rope=*/true, false, nullptr, Mode::kRun);
}
int minipic_reference_prerotated(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                                 const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                                 float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                 uint32_t flags, int32_t dtype, void* stream) {
  return run_attention(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, softmax_scale, out, workspace,
                       workspace_bytes, flags, dtype, stream, /*rope=*/false);
}

int minipic_decode_workspace_size(const minipic_batch* batch, int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(MINIPIC_ERR_INVALID_ARG, "bytes is NULL");
  int st = check_decode(batch, dtype);
  if (st) return st;
  DecodePlan pl;
  make_decode_plan(batch, &pl);
  *bytes = pl.bytes;
  return MINIPIC_OK;
}

int minipic_decode_attn(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                        const minipic_batch* batch, const float* cos_sin, int32_t max_pos, float softmax_scale,
                        void* out, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype,
                        void* stream) {
  return run_decode(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, softmax_scale, out, workspace,
                    workspace_bytes, flags, dtype, stream, /*rope=*/true);
}

int minipic_decode_prerotated(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                              const minipic_batch* batch, float softmax_scale, void* out, void* workspace,
                              size_t workspace_bytes, uint32_t flags, int32_t dtype, void* stream) {
  return run_decode(q, k_cache, v_cache, num_blocks, batch, nullptr, 0, softmax_scale, out, workspace,
                    workspace_bytes, flags, dtype, stream, /*rope=*/false);
}

int minipic_set_kernel_timing(int enable) {
  g_timer.on = enable != 0;
  g_timer.valid = false;
  g_timer.calls = 0;
  return MINIPIC_OK;
}

int minipic_kernel_times(float* ms) {
  if (!ms) return fail(MINIPIC_ERR_INVALID_ARG, "ms is NULL");
  if (!g_timer.on || !g_timer.valid) return fail(MINIPIC_ERR_INVALID_ARG, "no timed call (timing is off or no call yet)");
  const hipEvent_t* ev = &g_timer.ev[(size_t)((g_timer.calls - 1) % kTimedCalls) * 4];
  hipError_t e = hipEventSynchronize(ev[3]);
  for (int i = 0; i < 3 && e == hipSuccess; ++i) e = hipEventElapsedTime(&ms[i], ev[i], ev[i + 1]);
  if (e != hipSuccess) return hip_fail(e, "kernel timing events");
  return MINIPIC_OK;
}

int minipic_kernel_times_all(float* ms, int32_t max_calls, int32_t* num_calls) {
  if (!ms || !num_calls || max_calls < 0) return fail(MINIPIC_ERR_INVALID_ARG, "ms / num_calls NULL or max_calls < 0");
  if (!g_timer.on || !g_timer.valid) return fail(MINIPIC_ERR_INVALID_ARG, "no timed call (timing is off or no call yet)");
  const int64_t kept = g_timer.calls < kTimedCalls ? g_timer.calls : kTimedCalls;
  const int64_t n = kept < max_calls ? kept : max_calls;
  const hipEvent_t* last = &g_timer.ev[(size_t)((g_timer.calls - 1) % kTimedCalls) * 4];
  hipError_t e = hipEventSynchronize(last[3]);
  for (int64_t c = 0; c < n && e == hipSuccess; ++c) {
    const int64_t call = g_timer.calls - kept + c;   // oldest kept call first
    const hipEvent_t* ev = &g_timer.ev[(size_t)(call % kTimedCalls) * 4];
    for (int i = 0; i < 3 && e == hipSuccess; ++i) e = hipEventElapsedTime(&ms[3 * c + i], ev[i], ev[i + 1]);
  }
  if (e != hipSuccess) return hip_fail(e, "kernel timing events");
  *num_calls = (int32_t)n;
  return MINIPIC_OK;
}

}  // extern "C"
