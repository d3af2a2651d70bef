// Internal launch interface between the C ABI layer (api.cpp) and the kernel
// translation units. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Threads per decode split workgroup.
constexpr int kDecodeThreads = 256;
// Upper bound on split-KV work items per sequence (the combine kernel keeps
// one weight per split in LDS).
constexpr int kDecodeMaxSplits = 1024;

// Largest batch the balanced schedule takes (its prefix sums over the
// sequence lengths are one register per 64 sequences).
constexpr int kBalancedMaxB = 256;

struct DecodePlan {
  int split_rows;  // cache rows per split work item
  int splits;      // split work items per (b, kv head) in the grid; balanced:
                   // partial slots per (b, query head)
  // Balanced schedule (bf16 with per-sequence lengths, B <= kBalancedMaxB):
  // P workgroups, each at least C_min wave tiles of 4096/D rows.
  int balanced = 0;
  int P = 0, C_min = 0;
  // kv heads per unit of the balanced order: 1, or 4 for token-major pages
  // (a workgroup's four waves take four neighbouring heads of a tile)
  int hgs = 1;
};

struct DecodeArgs {
  bool bf16;
  const void *q, *k, *v;
  void *out;
  int B, Hq, Hkv, D, max_length;
  int position_id;          // used when seq_lens == nullptr
  const int32_t *seq_lens;  // device, may be null
  float scale;
  DecodePlan plan;
  float *ws_ml;  // [B][Hq][splits][2]  (running max, running sum)
  float *ws_o;   // [B][Hq][splits][D]  (unnormalised output)
  // Fused append (all null for a plain decode): k_new / v_new [B][Hkv][D]
  // are stored at each sequence's last valid row of the caches k_w / v_w
  // (the same memory as k / v) and attended to in the same launch.
  const void *k_new = nullptr, *v_new = nullptr;
  void *k_w = nullptr, *v_w = nullptr;
  // Rotary embedding in the fused append (null: none): fp32 [B][D] cos / sin
  // rows of each sequence's current position, applied to q and k_new.
  const float *rope_cos = nullptr, *rope_sin = nullptr;
  // Paged caches (bf16 only; null for a contiguous cache): k / v are
  // [num_pages][page_size][Hkv][D] (or head-major, below); block_table [B][max_blocks] gives the page
  // of every page_size rows of each sequence; max_length = max_blocks *
  // page_size and split_rows is a multiple of the wave tile.
  const int32_t *block_table = nullptr;
  int max_blocks = 0, page_size = 0, num_pages = 0;
  int head_major = 0;  // pages [num_pages][Hkv][page_size][D] instead
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
  const void *q, *k, *v;
  void *out;
  int B, Hq, Hkv, D, max_length, Lq, prefix_len;
  float scale;
  // Paged caches (null: contiguous): as for DecodeArgs; max_length =
  // max_blocks * page_size and page_size is a multiple of the 64-row tile.
  const int32_t *block_table = nullptr;
  int max_blocks = 0, page_size = 0, num_pages = 0;
  int head_major = 0;
};

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

struct TopkArgs {
  const float *q, *k, *v;
  float *out;
  int32_t *idx;
  int b, h, n, d, topk;
  bool causal = false;  // decoder form: keys j <= i, topk/2 most recent kept
};

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream);

// Streaming-read probe over n16 16-byte words of src; sink holds one 16-byte
// XOR per workgroup (1 <= workgroups <= 65536).
hipError_t launch_read_probe(const void *src, size_t n16, void *sink,
                             int workgroups, hipStream_t stream);

}  // namespace attn
