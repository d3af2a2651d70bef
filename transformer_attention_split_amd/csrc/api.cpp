// C ABI layer: argument validation, split planning and kernel enqueue.
//
// Every check below runs on host scalars before any HIP call, so an invalid
// call never touches the device. Nothing here allocates device memory or
// synchronises a stream.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/attn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

attn_status ok() {
  g_last_error.clear();
  return ATTN_OK;
}

attn_status hip_fail(hipError_t e, const char *what) {
  return fail(ATTN_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Product of extents fits comfortably in a signed 64-bit byte offset.
bool fits(std::initializer_list<double> dims) {
  double p = 1.0;
  for (double d : dims) p *= d;
  return p < 4.0e18;
}

// ---------------------------------------------------------------------------
// Decode planning. A work item is (kv head, sequence, split). The automatic
// choice aims for about kTargetBlocks workgroups (about half of them hold no
// rows for uniformly ragged lengths and exit at once) with a split length
// that is a whole number of rounds of the workgroup's four wave tiles (one
// wave tile is 8 KiB of K: 4096/D rows). At most attn::kDecodeMaxSplits
// splits per sequence: a smaller forced split_rows is raised to
// ceil(max_length / kDecodeMaxSplits). This plain grid runs fp32 caches,
// single sequences, batches without per-sequence lengths and batches of more
// than kBalancedMaxB sequences. The target was measured on 64 uniformly
// ragged sequences of up to 8192 rows (Hkv 8, D 128; before those went to the
// balanced schedule below), where it gives 896-row splits: 165 us per call
// against 169 us at 768 rows and 171 us at 1024 rows (fewer, longer splits
// leave a longer tail; more, shorter ones pay more per-workgroup start-up
// and combine work).
// ---------------------------------------------------------------------------
constexpr long kTargetBlocks = 5120;
constexpr long kCUs = 256;  // compute units of an MI355X

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

int row_quantum(int D) { return 4 * (4096 / D); }

int effective_split_rows(int max_length, int split_rows) {
  const int floor_rows = ceil_div(max_length, attn::kDecodeMaxSplits);
  return split_rows < floor_rows ? floor_rows : split_rows;
}

int auto_split_target(int B, int Hkv) {
  long items = (long)B * Hkv;
  long s = (kTargetBlocks + items - 1) / items;
  if (s < 1) s = 1;
  if (s > attn::kDecodeMaxSplits) s = attn::kDecodeMaxSplits;
  return (int)s;
}

attn::DecodePlan plan_decode(int B, int Hkv, int D, int max_length,
                             int L_bound, int split_rows) {
  attn::DecodePlan p{};
  if (split_rows > 0) {
    p.split_rows = effective_split_rows(max_length, split_rows);
  } else {
    const int q = row_quantum(D);
    int sr = ceil_div(L_bound, auto_split_target(B, Hkv));
    sr = ceil_div(sr, q) * q;
    // One round of the four wave tiles per workgroup only while the grid
    // fits one workgroup per CU; past that, two rounds. Measured on one
    // sequence (8 kv heads, D 128, graph replay, cold cache): at position
    // 8000, 504 one-round workgroups 14.2 us against 252 two-round ones
    // 12.9 us; at position 4000, 256 one-round workgroups 10.6 us against
    // 11.8 us.
    if (sr == q && (long)B * Hkv * ceil_div(L_bound, q) > kCUs) sr = 2 * q;
    p.split_rows = effective_split_rows(max_length, sr);
  }
  p.splits = ceil_div(L_bound, p.split_rows);
  if (p.splits < 1) p.splits = 1;
  return p;
}

// Balanced schedule (ragged bf16 batches of at most kBalancedMaxB sequences;
// the device side is described in decode.hip). Every wave is a worker that
// streams an equal run of the batch's wave tiles (at least C_min of them),
// across sequence ends, and writes one partial per piece it cuts: no merge
// of waves, no workgroup barrier. (With Hkv a multiple of 4 the unit is a
// group of four kv heads and the workgroup the worker, its wave w on head
// 4h + w: a quarter of the units for a quarter of the workers, so the same
// C_min and slot bound hold.) Two workgroups per CU, the split kernel's
// occupancy, so that every worker is resident from start to end: P = 4 *
// 512 workers (fewer when the batch at full length holds fewer runs of
// C_min tiles; P / 4 a multiple of 8, the XCD count, each of which takes a
// contiguous run of workers). Forcing split_rows sets C_min =
// ceil(split_rows / tile); otherwise C_min is 4 tiles or an eighth of a
// worker's share of the batch at full length, whichever is larger, so that
// batches of shorter sequences still occupy the grid while a partial
// (G*(D+2) floats) stays small against the rows it covers. C_min is at
// least ceil(n_max / (kDecodeMaxSplits - 1)), which bounds the pieces of
// one (b, kv head) by S = ceil(n_max / C_min) + 1 <= kDecodeMaxSplits
// (n_max: wave tiles of max_length rows). Per call on 64 uniformly ragged
// sequences of up to 8192 rows (Hkv 8, D 128): 159.1-159.7 us, against
// 168-172 us with one split per workgroup and 161-164 us with equal runs per
// workgroup whose four waves merge at every piece end.
struct BalancedPlan {
  bool ok;
  int P, C_min, S;
};

BalancedPlan plan_balanced(int B, int Hkv, int D, int max_length,
                           int split_rows) {
  BalancedPlan p{};
  const long tile = 4096 / D;
  const long n_max = ceil_div(max_length, tile);
  const long tt_max = (long)B * Hkv * n_max;
  p.P = 4 * 2 * (int)kCUs;
  // (one sequence has nothing to balance: its equal splits of the plain
  // grid finish together, while a run that straddles two kv heads takes
  // two pieces in turn: 13.3 against 15.7 us at 8001 rows, Hkv 8, D 128)
  if (B < 2 || B > attn::kBalancedMaxB || tt_max + p.P > INT_MAX) return p;
  long cmin;
  if (split_rows > 0) {
    cmin = ceil_div(split_rows, tile);
  } else {
    cmin = 4;
    const long share = ceil_div(tt_max, 8L * p.P);
    if (share > cmin) cmin = share;
  }
  const long floor_tiles = ceil_div(n_max, attn::kDecodeMaxSplits - 1);
  if (cmin < floor_tiles) cmin = floor_tiles;
  if (cmin > INT_MAX / p.P) cmin = INT_MAX / p.P;
  p.C_min = (int)cmin;
  // no more workers than runs of C_min tiles in the batch at full length
  const long need = (ceil_div(tt_max, cmin) + 31) / 32 * 32;
  if (need < p.P) p.P = (int)need;
  p.S = ceil_div(n_max, cmin) + 1;
  p.ok = true;
  return p;
}

// Upper bound on splits for any valid length <= max_length.
int max_splits(int B, int Hkv, int D, int max_length, int split_rows) {
  if (split_rows > 0)
    return ceil_div(max_length, effective_split_rows(max_length, split_rows));
  int a = auto_split_target(B, Hkv);
  int b = ceil_div(max_length, row_quantum(D));
  return a < b ? a : b;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t ws_ml_bytes(int B, int Hq, int S) {
  return align256((size_t)B * Hq * S * 2 * sizeof(float));
}
size_t ws_o_bytes(int B, int Hq, int S, int D) {
  return align256((size_t)B * Hq * S * D * sizeof(float));
}

}  // namespace

extern "C" {

const char *attn_status_str(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_E_ARG: return "ATTN_E_ARG: invalid argument";
    case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED: outside the supported set";
    case ATTN_E_WORKSPACE: return "ATTN_E_WORKSPACE: workspace missing or too small";
    case ATTN_E_HIP: return "ATTN_E_HIP: HIP runtime error";
  }
  return "unknown attn_status";
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

int attn_abi_version(void) { return 1; }

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D,
                                   int max_length, int split_rows) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || max_length < 1 || split_rows < 0)
    return 0;
  if (B == 0) return 0;
  if (!fits({(double)B, (double)Hq, (double)max_length, (double)D}))
    return 0;
  // a bound for both schedules (the balanced one is taken for ragged bf16
  // batches)
  int S = max_splits(B, Hkv, D, max_length, split_rows);
  const BalancedPlan bp = plan_balanced(B, Hkv, D, max_length, split_rows);
  if (bp.ok && bp.S > S) S = bp.S;
  return ws_ml_bytes(B, Hq, S) + ws_o_bytes(B, Hq, S, D);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points (fn names the entry point in error
// messages; k_new == nullptr: no append) and the launch arguments they imply;
// split lengths are rounded up to a multiple of row_multiple. Returns ATTN_OK
// with a.B == 0 for an empty batch (nothing to launch).
attn_status decode_check(const char *fn, attn_dtype dtype, const void *q, const void *k_new,
                 const void *v_new, const void *k_cache, const void *v_cache,
                 void *out, int B, int Hq, int Hkv, int D, int max_length,
                 int position_id, const int32_t *seq_lens, float scale,
                 int split_rows, void *workspace, size_t workspace_bytes,
                 int row_multiple, attn::DecodeArgs &a) {
  a = attn::DecodeArgs{};
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_E_ARG, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || B > 65535)
    return fail(ATTN_E_ARG, "%s: B=%d outside [0, 65535]", fn, B);
  if (Hq < 1 || Hkv < 1 || Hkv > 65535)
    return fail(ATTN_E_ARG, "%s: Hq=%d Hkv=%d must be >= 1 (Hkv <= 65535)", fn, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(ATTN_E_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(ATTN_E_UNSUPPORTED, "%s: group size Hq/Hkv=%d not in {1,2,4,8}", fn, G);
  if (D < 1) return fail(ATTN_E_ARG, "%s: D=%d", fn, D);
  if (D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  if (max_length < 1)
    return fail(ATTN_E_ARG, "%s: max_length=%d must be >= 1", fn, max_length);
  if (!fits({(double)B, (double)Hkv, (double)max_length, (double)D, 4.0}) ||
      !fits({(double)B, (double)Hq, (double)max_length, (double)D, 4.0}))
    return fail(ATTN_E_ARG, "%s: cache extents overflow", fn);
  if (seq_lens == nullptr && (position_id < 0 || position_id >= max_length))
    return fail(ATTN_E_ARG, "%s: position_id=%d outside [0, max_length=%d)", fn,
                position_id, max_length);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_E_ARG, "%s: scale must be finite and > 0", fn);
  if (split_rows < 0)
    return fail(ATTN_E_ARG, "%s: split_rows=%d < 0", fn, split_rows);
  if (B == 0) return ok();  // empty batch: nothing is read or written
  if (!q || !k_cache || !v_cache || !out)
    return fail(ATTN_E_ARG, "%s: null data pointer", fn);
  if (k_new && (!v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
    return fail(ATTN_E_ARG, "%s: k_new / v_new must be non-null and 16-byte aligned", fn);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16))
    return fail(ATTN_E_ARG, "%s: data pointers must be 16-byte aligned", fn);
  if (seq_lens && !aligned(seq_lens, 4))
    return fail(ATTN_E_ARG, "%s: seq_lens must be 4-byte aligned", fn);
  const size_t need =
      attn_decode_workspace_bytes(B, Hq, Hkv, D, max_length, split_rows);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (!aligned(workspace, 256))
    return fail(ATTN_E_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);

  const int L_bound = seq_lens ? max_length : position_id + 1;
  a.bf16 = dtype == ATTN_BF16;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.max_length = max_length;
  a.position_id = position_id;
  a.seq_lens = seq_lens;
  a.scale = scale;
  a.plan = plan_decode(B, Hkv, D, max_length, L_bound, split_rows);
  if (seq_lens && dtype == ATTN_BF16) {
    const BalancedPlan bp = plan_balanced(B, Hkv, D, max_length, split_rows);
    if (bp.ok) {
      a.plan.balanced = 1;
      a.plan.P = bp.P;
      a.plan.C_min = bp.C_min;
      a.plan.splits = bp.S;  // pieces start at wave-tile rows: no page straddles
      // Groups of four kv heads: a workgroup's four waves take four
      // neighbouring heads of the same tiles (the plan's C_min and slot bound
      // hold: a quarter of the units, a quarter of the workers). Token-major
      // pages keep the heads of a token side by side, so the four waves read
      // 1 KiB contiguous of the same token rows (168.3 against 184.4 us with
      // one wave per head, ragged batch in 64-row pages); contiguous caches
      // gain 1-2 % (ragged batch 159.3 against 160.9 us, sorted 158.5
      // against 162.3 us), and every layout keeps one plan.
      if (Hkv % 4 == 0) a.plan.hgs = 4;
    }
  }
  if (!a.plan.balanced && a.plan.split_rows % row_multiple != 0) {  // fewer splits: still fits
    a.plan.split_rows = ceil_div(a.plan.split_rows, row_multiple) * row_multiple;
    a.plan.splits = ceil_div(L_bound, a.plan.split_rows);
  }
  char *ws = static_cast<char *>(workspace);
  a.ws_ml = reinterpret_cast<float *>(ws);
  ws += ws_ml_bytes(B, Hq, a.plan.splits);
  a.ws_o = reinterpret_cast<float *>(ws);
  if (k_new) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_w = const_cast<void *>(k_cache);
    a.v_w = const_cast<void *>(v_cache);
  }
  return ok();
}

attn_status decode_impl(const char *fn, attn_dtype dtype, const void *q, const void *k_new,
                const void *v_new, const void *k_cache, const void *v_cache,
                void *out, int B, int Hq, int Hkv, int D, int max_length,
                int position_id, const int32_t *seq_lens, float scale,
                int split_rows, void *workspace, size_t workspace_bytes,
                void *stream, const float *rope_cos = nullptr,
                const float *rope_sin = nullptr) {
  attn::DecodeArgs a;
  const attn_status st = decode_check(fn, dtype, q, k_new, v_new, k_cache, v_cache,
                              out, B, Hq, Hkv, D, max_length, position_id,
                              seq_lens, scale, split_rows, workspace,
                              workspace_bytes, 1, a);
  if (st != ATTN_OK || a.B == 0) return st;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  hipError_t e = attn::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // namespace

extern "C" {

attn_status attn_decode(attn_dtype dtype, const void *q, const void *k_cache,
                const void *v_cache, void *out, int B, int Hq, int Hkv, int D,
                int max_length, int position_id, const int32_t *seq_lens,
                float scale, int split_rows, void *workspace,
                size_t workspace_bytes, void *stream) {
  return decode_impl("attn_decode", dtype, q, nullptr, nullptr, k_cache,
                     v_cache, out, B, Hq, Hkv, D, max_length, position_id,
                     seq_lens, scale, split_rows, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free decode: the split partials live in a file-scope device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy of the array (kScratchBytes) until the process ends. In host code
// the array's name is not a device address: the address of each GPU's copy
// is looked up once, with that GPU current, and only that address is passed
// to the kernels.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
void *g_scratch_dev[kMaxDevices];  // device address of scratch, per GPU
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

extern "C" {

attn_status attn_decode_noalloc(attn_dtype dtype, const void *q,
                                const void *k_cache, const void *v_cache,
                                void *out, int B, int Hq, int Hkv, int D,
                                int max_length, int position_id,
                                const int32_t *seq_lens, float scale,
                                int split_rows, void *stream) {
  const char *fn = "attn_decode_noalloc";
  // Every argument check first, on host scalars: a stand-in workspace
  // address (never dereferenced) and the scratch size.
  {
    attn::DecodeArgs probe;
    const size_t need = attn_decode_workspace_bytes(
        B, Hq, Hkv, D, max_length, split_rows < 0 ? 0 : split_rows);
    if (need > kScratchBytes)
      return fail(ATTN_E_WORKSPACE,
                  "%s: these sizes need %zu bytes of split scratch, the static "
                  "scratch holds %zu (use attn_decode with a workspace)",
                  fn, need, kScratchBytes);
    const attn_status st = decode_check(
        fn, dtype, q, nullptr, nullptr, k_cache, v_cache, out, B, Hq, Hkv, D,
        max_length, position_id, seq_lens, scale, split_rows,
        reinterpret_cast<void *>(uintptr_t(256)), kScratchBytes, 1, probe);
    if (st != ATTN_OK || probe.B == 0) return st;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_E_UNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxDevices);
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (sdev != dev)
      return fail(ATTN_E_ARG, "%s: stream belongs to device %d, device %d is current",
                  fn, (int)sdev, dev);
  }
  std::call_once(g_scratch_once[dev], [dev]() {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_dev[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess)
    return hip_fail(g_scratch_err[dev], "attn_decode_noalloc: scratch address");
  return decode_impl(fn, dtype, q, nullptr, nullptr, k_cache, v_cache, out, B,
                     Hq, Hkv, D, max_length, position_id, seq_lens, scale,
                     split_rows, g_scratch_dev[dev], kScratchBytes, stream);
}

attn_status attn_decode_append(attn_dtype dtype, const void *q, const void *k_new,
                       const void *v_new, void *k_cache, void *v_cache,
                       void *out, int B, int Hq, int Hkv, int D, int max_length,
                       int position_id, const int32_t *seq_lens, float scale,
                       int split_rows, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (B > 0 && (!k_new || !v_new))
    return fail(ATTN_E_ARG, "attn_decode_append: null k_new / v_new");
  return decode_impl("attn_decode_append", dtype, q, k_new, v_new, k_cache,
                     v_cache, out, B, Hq, Hkv, D, max_length, position_id,
                     seq_lens, scale, split_rows, workspace, workspace_bytes,
                     stream);
}

attn_status attn_decode_append_rope(attn_dtype dtype, const void *q, const void *k_new,
                            const void *v_new, const float *rope_cos,
                            const float *rope_sin, void *k_cache, void *v_cache,
                            void *out, int B, int Hq, int Hkv, int D,
                            int max_length, int position_id,
                            const int32_t *seq_lens, float scale, int split_rows,
                            void *workspace, size_t workspace_bytes,
                            void *stream) {
  const char *fn = "attn_decode_append_rope";
  if (B > 0 && (!k_new || !v_new || !rope_cos || !rope_sin))
    return fail(ATTN_E_ARG, "%s: null k_new / v_new / rope_cos / rope_sin", fn);
  if (B > 0 && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16)))
    return fail(ATTN_E_ARG, "%s: rope_cos / rope_sin must be 16-byte aligned", fn);
  return decode_impl(fn, dtype, q, k_new, v_new, k_cache, v_cache, out, B, Hq,
                     Hkv, D, max_length, position_id, seq_lens, scale,
                     split_rows, workspace, workspace_bytes, stream, rope_cos,
                     rope_sin);
}


attn_status attn_decode_paged(attn_dtype dtype, const void *q, const void *k_pages,
                      const void *v_pages, const int32_t *block_table,
                      int max_blocks, int page_size, int num_pages,
                      attn_page_layout page_layout, void *out,
                      int B, int Hq, int Hkv, int D, int position_id,
                      const int32_t *seq_lens, float scale, int split_rows,
                      void *workspace, size_t workspace_bytes, void *stream) {
  const char *fn = "attn_decode_paged";
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_E_ARG, "%s: unknown dtype %d", fn, dtype);
  if (dtype != ATTN_BF16)
    return fail(ATTN_E_UNSUPPORTED, "%s: only ATTN_BF16 is supported", fn);
  if (D != 64 && D != 128)
    return fail(D < 1 ? ATTN_E_ARG : ATTN_E_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  const int tile = 4096 / D;  // rows of one wave tile
  if (page_size < 1 || max_blocks < 1 || num_pages < 1)
    return fail(ATTN_E_ARG, "%s: page_size=%d max_blocks=%d num_pages=%d must be >= 1",
                fn, page_size, max_blocks, num_pages);
  if (page_layout != ATTN_PAGES_TOKEN_MAJOR && page_layout != ATTN_PAGES_HEAD_MAJOR)
    return fail(ATTN_E_ARG, "%s: unknown page_layout %d", fn, page_layout);
  if (page_size % tile != 0 || page_size > 65536)
    return fail(ATTN_E_UNSUPPORTED, "%s: page_size=%d is not a multiple of %d in [%d, 65536]",
                fn, page_size, tile, tile);
  if ((long long)max_blocks * page_size > 0x7fffffffLL ||
      !fits({(double)num_pages, (double)page_size, (double)Hkv, (double)D, 2.0}))
    return fail(ATTN_E_ARG, "%s: page extents overflow", fn);
  const int max_length = max_blocks * page_size;
  if (B > 0 && !block_table)
    return fail(ATTN_E_ARG, "%s: null block_table", fn);
  if (block_table && !aligned(block_table, 4))
    return fail(ATTN_E_ARG, "%s: block_table must be 4-byte aligned", fn);
  // The remaining checks are those of the logical cache
  // [B][Hkv][max_length][D]; split lengths become multiples of the wave tile
  // so that no tile straddles a page.
  attn::DecodeArgs a;
  const attn_status st = decode_check(fn, dtype, q, nullptr, nullptr, k_pages, v_pages,
                              out, B, Hq, Hkv, D, max_length, position_id,
                              seq_lens, scale, split_rows, workspace,
                              workspace_bytes, tile, a);
  if (st != ATTN_OK || a.B == 0) return st;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.head_major = page_layout == ATTN_PAGES_HEAD_MAJOR;
  hipError_t e = attn::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by the prefill entry points; a.B == 0 on return: nothing to
// launch.
attn_status prefill_check(const char *fn, attn_dtype dtype, const void *q, const void *k,
                  const void *v, void *out, int B, int Hq, int Hkv, int D,
                  int max_length, int Lq, int prefix_len, float scale,
                  attn::PrefillArgs &a) {
  a = attn::PrefillArgs{};
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_E_ARG, "%s: unknown dtype %d", fn, dtype);
  if (dtype != ATTN_BF16)
    return fail(ATTN_E_UNSUPPORTED, "%s: only ATTN_BF16 is supported", fn);
  if (B < 0 || B > 65535)
    return fail(ATTN_E_ARG, "%s: B=%d outside [0, 65535]", fn, B);
  if (Hq < 1 || Hq > 65535 || Hkv < 1)
    return fail(ATTN_E_ARG, "%s: Hq=%d Hkv=%d must be >= 1 (Hq <= 65535)", fn, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(ATTN_E_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (D < 1) return fail(ATTN_E_ARG, "%s: D=%d", fn, D);
  if (D != 64 && D != 128)
    return fail(ATTN_E_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  if (max_length < 1 || Lq < 0 || prefix_len < 0)
    return fail(ATTN_E_ARG, "%s: max_length=%d Lq=%d prefix_len=%d", fn,
                max_length, Lq, prefix_len);
  if ((long long)prefix_len + Lq > max_length)
    return fail(ATTN_E_ARG, "%s: prefix_len+Lq=%lld exceeds max_length=%d", fn,
                (long long)prefix_len + Lq, max_length);
  if (!fits({(double)B, (double)Hkv, (double)max_length, (double)D, 2.0}) ||
      !fits({(double)B, (double)Hq, (double)max_length, (double)D, 2.0}))
    return fail(ATTN_E_ARG, "%s: extents overflow", fn);
  // The kernel addresses the rows [0, prefix_len + Lq) of one kv head with
  // 32-bit byte offsets.
  if (((long long)prefix_len + Lq) * D * 2 > 0x7fffffffLL)
    return fail(ATTN_E_UNSUPPORTED, "%s: prefix_len+Lq=%lld rows of %d bytes exceed 2^31 bytes",
                fn, (long long)prefix_len + Lq, 2 * D);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_E_ARG, "%s: scale must be finite and > 0", fn);
  if (B == 0 || Lq == 0) return ok();  // nothing is read or written
  if (!q || !k || !v || !out)
    return fail(ATTN_E_ARG, "%s: null data pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(ATTN_E_ARG, "%s: data pointers must be 16-byte aligned", fn);
  a = attn::PrefillArgs{q, k, v, out, B, Hq, Hkv, D, max_length, Lq, prefix_len, scale};
  return ok();
}

}  // namespace

extern "C" {

attn_status attn_prefill(attn_dtype dtype, const void *q, const void *k_cache,
                 const void *v_cache, void *out, int B, int Hq, int Hkv, int D,
                 int max_length, int Lq, int prefix_len, float scale,
                 void *stream) {
  attn::PrefillArgs a;
  const attn_status st = prefill_check("attn_prefill", dtype, q, k_cache, v_cache, out,
                               B, Hq, Hkv, D, max_length, Lq, prefix_len, scale, a);
  if (st != ATTN_OK || a.B == 0) return st;
  hipError_t e = attn::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attn_prefill launch");
  return ok();
}

attn_status attn_prefill_paged(attn_dtype dtype, const void *q, const void *k_pages,
                       const void *v_pages, const int32_t *block_table,
                       int max_blocks, int page_size, int num_pages,
                       attn_page_layout page_layout, void *out, int B, int Hq, int Hkv, int D,
                       int Lq, int prefix_len, float scale, void *stream) {
  const char *fn = "attn_prefill_paged";
  if (page_size < 1 || max_blocks < 1 || num_pages < 1)
    return fail(ATTN_E_ARG, "%s: page_size=%d max_blocks=%d num_pages=%d must be >= 1",
                fn, page_size, max_blocks, num_pages);
  const int tile = D == 128 ? 32 : 64;  // keys per kernel tile (8 KiB of K)
  if (page_size % tile != 0 || page_size > 65536)
    return fail(ATTN_E_UNSUPPORTED,
                "%s: page_size=%d must be a multiple of %d rows and <= 65536", fn,
                page_size, tile);
  if (page_layout != ATTN_PAGES_TOKEN_MAJOR && page_layout != ATTN_PAGES_HEAD_MAJOR)
    return fail(ATTN_E_ARG, "%s: page_layout=%d", fn, page_layout);
  if ((long long)max_blocks * page_size > 0x7fffffffLL)
    return fail(ATTN_E_ARG, "%s: max_blocks*page_size exceeds 2^31-1", fn);
  if (Hkv >= 1 && D >= 1 &&
      !fits({(double)num_pages, (double)page_size, (double)Hkv, (double)D, 2.0}))
    return fail(ATTN_E_ARG, "%s: page pool extents overflow", fn);
  attn::PrefillArgs a;
  const attn_status st = prefill_check(fn, dtype, q, k_pages, v_pages, out, B, Hq, Hkv,
                               D, max_blocks * page_size, Lq, prefix_len, scale, a);
  if (st != ATTN_OK || a.B == 0) return st;
  if (!block_table) return fail(ATTN_E_ARG, "%s: null block_table", fn);
  if (!aligned(block_table, 4))
    return fail(ATTN_E_ARG, "%s: block_table must be 4-byte aligned", fn);
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.head_major = page_layout == ATTN_PAGES_HEAD_MAJOR;
  hipError_t e = attn::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

static attn_status topk_impl(const char *fn, bool causal, const float *q, const float *k,
                     const float *v, float *out, int32_t *idx_out, int b, int h,
                     int n, int d, int topk, void *stream) {
  if (b < 0 || b > 65535 || h < 0 || h > 65535)
    return fail(ATTN_E_ARG, "%s: b=%d h=%d outside [0, 65535]", fn, b, h);
  if (d < 1) return fail(ATTN_E_ARG, "%s: d=%d", fn, d);
  if (d != 64) return fail(ATTN_E_UNSUPPORTED, "%s: d=%d, only 64", fn, d);
  if (n < 1) return fail(ATTN_E_ARG, "%s: n=%d must be >= 1", fn, n);
  if (n > 1024) return fail(ATTN_E_UNSUPPORTED, "%s: n=%d > 1024", fn, n);
  if (topk < 1 || topk > n)
    return fail(ATTN_E_ARG, "%s: topk=%d outside [1, n=%d]", fn, topk, n);
  if ((int64_t)b * h * ((n + 15) / 16) > (int64_t)1 << 23)
    return fail(ATTN_E_UNSUPPORTED,
                "%s: b*h*ceil(n/16)=%lld workgroups > 2^23", fn,
                (long long)b * h * ((n + 15) / 16));
  if (b == 0 || h == 0) return ok();  // nothing is read or written
  if (!q || !k || !v || !out)
    return fail(ATTN_E_ARG, "%s: null data pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(out, 16))
    return fail(ATTN_E_ARG, "%s: data pointers must be 16-byte aligned", fn);
  if (idx_out && !aligned(idx_out, 4))
    return fail(ATTN_E_ARG, "%s: idx_out must be 4-byte aligned", fn);
  attn::TopkArgs a{q, k, v, out, idx_out, b, h, n, d, topk, causal};
  hipError_t e = attn::launch_topk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

attn_status attn_topk(const float *q, const float *k, const float *v, float *out,
              int32_t *idx_out, int b, int h, int n, int d, int topk,
              void *stream) {
  return topk_impl("attn_topk", false, q, k, v, out, idx_out, b, h, n, d, topk, stream);
}

attn_status attn_topk_causal(const float *q, const float *k, const float *v, float *out,
                     int32_t *idx_out, int b, int h, int n, int d, int topk,
                     void *stream) {
  return topk_impl("attn_topk_causal", true, q, k, v, out, idx_out, b, h, n, d, topk,
                   stream);
}

attn_status attn_read_probe(const void *src, size_t bytes, void *sink,
                    size_t sink_bytes, int workgroups, void *stream) {
  const char *fn = "attn_read_probe";
  if (workgroups < 1 || workgroups > 65536)
    return fail(ATTN_E_ARG, "%s: workgroups=%d outside [1, 65536]", fn, workgroups);
  if (bytes % 16 != 0)
    return fail(ATTN_E_ARG, "%s: bytes=%zu is not a multiple of 16", fn, bytes);
  if (sink_bytes < (size_t)16 * (size_t)workgroups)
    return fail(ATTN_E_ARG, "%s: sink holds %zu bytes, needs 16 * %d", fn,
                sink_bytes, workgroups);
  if (!sink || (bytes > 0 && !src))
    return fail(ATTN_E_ARG, "%s: null pointer", fn);
  if (!aligned(src, 16) || !aligned(sink, 16))
    return fail(ATTN_E_ARG, "%s: src and sink must be 16-byte aligned", fn);
  hipError_t e = attn::launch_read_probe(src, bytes / 16, sink, workgroups,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // extern "C"
