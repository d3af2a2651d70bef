// Split-KV single-token decode over a static KV cache (gfx950, wave64).
//
// Operation: "MiniCPM4 forward_step Attention Performance Fix", §3 and §4.1 —
// the query of the new token attends only to cache rows [0, position_id]
// (or [0, seq_len) per sequence); the slice bound replaces the mask, so the
// work and the bytes read are proportional to the valid length (§2.4 cost
// table). Query head h reads kv head h / G (G = Hq/Hkv), so each K and V row
// is read once and serves the whole group of G query heads.
//
// Ragged bf16 batches of 2 to kBalancedMaxB sequences run the balanced
// schedule described below its helpers: every wave streams an equal run of
// the batch's tiles. Otherwise:
// work item = (kv head g, sequence b, split s) = cache rows
// [s*split_rows, min((s+1)*split_rows, L_b)). The grid is (Hkv, B, splits),
// dispatched x fastest. With one length for the whole batch the split index
// varies slowest: the round-robin dispatch over the 8 XCDs spreads every
// split index evenly over them, the short last splits come last and splits
// that hold no rows exit at once. With per-sequence lengths (up to
// kReorderMaxB sequences) the dispatch order is remapped on the device: the
// full splits of all sequences first, then the partial last splits, then
// one unit per zero-length sequence (it writes the zero rows), then idle
// workgroups. Full splits all cost the same, so the partial ones fill the
// gaps at the end instead of a late full split running alone.
//
// bf16 (decode_bf16_kernel): each of the 4 waves walks its own tiles of BN
// rows (BN*D*2 = 8 KiB of K and of V per tile) with non-temporal 16-byte
// loads, and runs both products on the bf16 matrix cores — the kernel stays
// bound by HBM; the matrix cores only take the multiply-adds off the vector
// ALUs, which would otherwise need more issue slots per byte than a CU has:
//   Sᵀ = K·Qᵀ  v_mfma_f32_16x16x32_bf16, A = 16 K rows (loaded as whole
//              rows and laid out through the wave's LDS K tile),
//              B = the G query heads of the group (columns >= G zero);
//              lane (q, lane-group) receives 4 keys of query q;
//   softmax    online, exp2 domain (scale*log2 e applied to fp32 scores); the
//              running max is reduced over the 4 lanes that share a query;
//              the output is rescaled only when some running max moved;
//   Oᵀ += Vᵀ·Pᵀ  V rows are transposed through this wave's LDS tile (eight
//              rows per lane packed into 16-byte writes), P is rounded to
//              bf16 and stays in registers.
// fp32 (decode_f32_kernel): vector-ALU form — each cache row is read by a
// group of D/4 lanes (16-byte loads), dot products reduced with DPP row
// operations, online softmax per group.
//
// Both end the same way: the workgroup merges its waves / row groups (under
// the balanced schedule every wave ends on its own, no merge) and either
// writes the output directly (the sequence has a single split) or writes
// one partial (running max, running sum, unnormalised output) per query
// head to the workspace. decode_combine_kernel then merges the
// partials of every multi-split sequence (log-sum-exp: each partial weighted
// by exp of its running max less the largest), divides by the total sum and
// casts to the output type. (Merging inside the
// split kernel, in the last workgroup of each (b, g) to finish, measured
// twice as slow with agent-scope fences, and no faster than the second
// launch with the partials written and read through agent-scope stores and
// loads: the write-through wait, the counter's round trip and the partial
// reads then sit on the last workgroup's path.)
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ldnt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Rotary position embedding, rotate-half convention: element j of a row is
// paired with j + D/2, out_j = x_j·cos_j + r_j·sin_j with r_j = -x_{j+D/2}
// for j < D/2 and x_{j-D/2} otherwise; fp32, one fma per element.
// rope_bf16x8: x = 8 bf16 elements j0..j0+7, p = their partners, c / s the
// cos / sin values of j0..j0+7, lo = (j0 < D/2); one rounding to bf16.
__device__ __forceinline__ float rope1(float x, float p, float c, float s, bool lo) {
  return fmaf(x, c, (lo ? -p : p) * s);
}
__device__ __forceinline__ u32x4_t rope_bf16x8(u32x4_t x, u32x4_t p, const float *c,
                                               const float *s, bool lo) {
  const float4 c0 = *reinterpret_cast<const float4 *>(c);
  const float4 c1 = *reinterpret_cast<const float4 *>(c + 4);
  const float4 s0 = *reinterpret_cast<const float4 *>(s);
  const float4 s1 = *reinterpret_cast<const float4 *>(s + 4);
  const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  u32x4_t r;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    r[w] = pack_bf16x2(rope1(bf16lo(x[w]), bf16lo(p[w]), cc[2 * w], ss[2 * w], lo),
                       rope1(bf16hi(x[w]), bf16hi(p[w]), cc[2 * w + 1], ss[2 * w + 1], lo));
  return r;
}
// the same for 4 fp32 elements (no rounding)
__device__ __forceinline__ u32x4_t rope_f32x4(u32x4_t x, u32x4_t p, const float *c,
                                              const float *s, bool lo) {
  const float4 cv = *reinterpret_cast<const float4 *>(c);
  const float4 sv = *reinterpret_cast<const float4 *>(s);
  const float cc[4] = {cv.x, cv.y, cv.z, cv.w}, ss[4] = {sv.x, sv.y, sv.z, sv.w};
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = __float_as_uint(rope1(__uint_as_float(x[e]), __uint_as_float(p[e]), cc[e], ss[e], lo));
  return r;
}

struct Item {
  int L;        // valid rows of the sequence
  int row0;     // first row of this split
  int row1;     // one past the last row of this split
  int n_split;  // splits of this sequence that hold rows
};

__device__ __forceinline__ Item make_item(const int32_t *seq_lens, int b,
                                          int position_id, int max_length,
                                          int split_rows, int s) {
  Item it;
  if (seq_lens == nullptr) {
    it.L = position_id + 1;
  } else {
    int L = seq_lens[b];
    it.L = L < 0 ? 0 : (L > max_length ? max_length : L);
  }
  it.row0 = s * split_rows;
  it.row1 = min(it.row0 + split_rows, it.L);
  it.n_split = (it.L + split_rows - 1) / split_rows;
  return it;
}

// ---------------------------------------------------------------------------
// Work units
// ---------------------------------------------------------------------------
constexpr int kReorderMaxB = 256;

struct Unit {
  int g, b, s;  // kv head, sequence (-1: no work), split
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  return (int)wave_inclusive_scan((uint32_t)x, lane);  // (counts are >= 0)
}

// The work unit of this workgroup (the orders are described at the top).
__device__ __forceinline__ Unit locate_unit(const int32_t *seq_lens, int B,
                                            int Hkv, int max_length,
                                            int split_rows) {
  Unit u{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  if (seq_lens == nullptr || B > kReorderMaxB) return u;
  const int i = blockIdx.x + Hkv * (blockIdx.y + B * blockIdx.z);
  u.g = i % Hkv;
  int r = i / Hkv;  // rank among the (sequence, split) units; wave-uniform
  const int lane = threadIdx.x % 64;
  int Ls[kReorderMaxB / 64];
#pragma unroll
  for (int c = 0; c < kReorderMaxB / 64; ++c) {
    const int bi = 64 * c + lane;
    int L = bi < B ? seq_lens[bi] : 0;
    Ls[c] = L < 0 ? 0 : (L > max_length ? max_length : L);
  }
  for (int cat = 0; cat < 3; ++cat) {  // full splits, partial splits, zero rows
#pragma unroll
    for (int c = 0; c < kReorderMaxB / 64; ++c) {
      if (64 * c >= B) break;
      const int L = Ls[c];
      const int cnt = cat == 0   ? L / split_rows
                      : cat == 1 ? (L % split_rows != 0)
                                 : (64 * c + lane < B && L == 0);
      const int incl = wave_incl_scan(cnt, lane);
      const int tot = __shfl(incl, 63);
      if (r < tot) {
        const int ln = __ffsll((unsigned long long)__ballot(incl > r)) - 1;
        u.b = 64 * c + ln;
        const int excl = __shfl(incl - cnt, ln);
        const int Lb = __shfl(L, ln);
        u.s = cat == 0 ? r - excl : cat == 1 ? Lb / split_rows : 0;
        return u;
      }
      r -= tot;
    }
  }
  u.b = -1;
  return u;
}

// ---------------------------------------------------------------------------
// Balanced schedule (bf16, per-sequence lengths, B <= kBalancedMaxB)
// ---------------------------------------------------------------------------
// The work of the batch is the list of wave tiles (BN rows) of every
// (sequence b, kv head g) in the order (b, g, tile): n_b = ceil(L_b / BN)
// tiles per kv head of sequence b, TT = Hkv * sum_b n_b in all. Every wave
// is a worker: worker u of the P launched (four per workgroup) takes the
// tiles [u*C, (u+1)*C), C = max(C_min, ceil(TT / P)), so every wave streams
// the same number of rows whatever the lengths, and a long sequence no
// longer ends the launch alone; no wave waits for another. A range cuts one
// or more (b, g) into pieces. A (b, g) inside one range is finished there;
// the others leave one partial per piece, in slot u - first(b, g),
// first(b, g) = floor(start(b, g) / C), start(b, g) = Hkv * P_b + g * n_b
// (P_b: the tiles of the sequences before b), which the combine kernel finds
// from the same lengths.
__device__ __forceinline__ int clamp_len(int L, int max_length) {
  return L < 0 ? 0 : (L > max_length ? max_length : L);
}

struct BatchTiles {
  int len[kBalancedMaxB / 64];   // clamped length of sequence 64c + lane
  int cnt[kBalancedMaxB / 64];   // n_b of sequence 64c + lane
  int incl[kBalancedMaxB / 64];  // sum of n_b' over b' <= 64c + lane
  int total;                     // sum of n_b over the batch (wave-uniform)
};

__device__ __forceinline__ BatchTiles batch_tiles(const int32_t *seq_lens,
                                                  int B, int max_length,
                                                  int BN) {
  const int lane = threadIdx.x % 64;
  BatchTiles t;
  t.total = 0;
#pragma unroll
  for (int c = 0; c < kBalancedMaxB / 64; ++c) {
    const int bi = 64 * c + lane;
    t.len[c] = bi < B ? clamp_len(seq_lens[bi], max_length) : 0;
    t.cnt[c] = (t.len[c] + BN - 1) / BN;
    t.incl[c] = t.total;
    if (64 * c < B) {  // (uniform)
      t.incl[c] += wave_incl_scan(t.cnt[c], lane);
      t.total = __builtin_amdgcn_readlane(t.incl[c], 63);  // scalar
    }
  }
  return t;
}

// Value of lane (b % 64) of chunk b / 64 (b wave-uniform): a lane read, no
// memory access.
__device__ __forceinline__ int seq_value(const int (&v)[kBalancedMaxB / 64], int b) {
  const int c = b >> 6;
  const int x = c == 0 ? v[0] : c == 1 ? v[1] : c == 2 ? v[2] : v[3];
  return __builtin_amdgcn_readlane(x, b & 63);
}

// Tiles per workgroup (the host keeps TT + P and P * C_min below 2^31).
__device__ __forceinline__ int chunk_tiles(int TT, int P, int C_min) {
  const int c = (TT + P - 1) / P;
  return c > C_min ? c : C_min;
}

template <bool BF16>
__device__ __forceinline__ void store_out(void *outp, size_t idx, float x) {
  if constexpr (BF16) {
    static_cast<uint16_t *>(outp)[idx] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
  } else {
    static_cast<float *>(outp)[idx] = x;
  }
}

// Shared ending. fin_m/fin_l/fin_o (LDS) hold this workgroup's merged
// running max, sum and unnormalised output of the G query heads of (b, g).
// A piece that is the whole (b, g) (direct) is finished here; otherwise the
// partial is written to slot s of (b, g) for the combine kernel.
template <bool BF16, int D, int G, int NT>
__device__ __forceinline__ void finish(const float *fin_m, const float *fin_l,
                                       const float *fin_o, bool direct,
                                       int b, int g, int s, int Hq,
                                       int splits, void *outp, float *ws_ml,
                                       float *ws_o) {
  const int tid = threadIdx.x;
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  if (direct) {
    for (int i = tid; i < G * D; i += NT) {
      const int h = i / D, d = i % D;
      store_out<BF16>(outp, (head0 + h) * D + d, fin_o[h * D + d] / fin_l[h]);
    }
    return;
  }
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, d = i % D;
    ws_o[((head0 + h) * splits + s) * D + d] = fin_o[h * D + d];
  }
  if (tid < G) {
    float *ml = ws_ml + ((head0 + tid) * splits + s) * 2;
    ml[0] = fin_m[tid];
    ml[1] = fin_l[tid];
  }
}

template <bool BF16, int D, int G, int NT>
__device__ __forceinline__ void write_zero_rows(void *outp, int b, int g,
                                                int Hq) {
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  for (int i = threadIdx.x; i < G * D; i += NT) store_out<BF16>(outp, head0 * D + i, 0.f);
}

// ---------------------------------------------------------------------------
// bf16: matrix-core form
// ---------------------------------------------------------------------------
constexpr int kThreads = kDecodeThreads;  // 4 waves

template <int D>
struct Bf16Tile {
  static constexpr int BN = 4096 / D;      // rows per wave tile (8 KiB of K)
  static constexpr int KS = D / 32;        // k-steps of K·Qᵀ
  static constexpr int NDB = D / 16;       // 16-wide output blocks
  static constexpr int NKB = BN / 16;      // 16-row blocks per tile
  static constexpr int SV = BN + 4;        // Vᵀ row stride in LDS (elements)
  static constexpr int NOCT = BN / 8;      // 8-row groups per tile
  static constexpr int VT_BYTES = D * SV * 2;
  static_assert(NOCT * (D / 8) == 64, "one V transpose item per lane");
};

// A piece of work: rows [row0, row1) of kv head g of sequence b (valid length
// L); direct: the piece is the whole (b, g), whose output it writes, else its
// partial goes to slot `slot` of (b, g).
struct Piece {
  int b, g, row0, row1, L, slot, direct;
};

// MODE: 0 = contiguous cache, 1 = contiguous cache with the fused append,
// 2 = paged cache, 3 = fused append with the rotary embedding of the query
// and the new key. SOLO: the balanced schedule, every wave a worker of its
// own (below); otherwise one work unit per workgroup, its four waves taking
// every fourth tile and merging at the end.
template <int D, int G, int MODE, bool SOLO>
__global__ __launch_bounds__(kThreads, 2) void decode_bf16_kernel(
    const uint16_t *__restrict__ qg, const uint16_t *__restrict__ kg,
    const uint16_t *__restrict__ vg, const int32_t *__restrict__ seq_lens,
    int position_id, void *__restrict__ outp, float *__restrict__ ws_ml,
    float *__restrict__ ws_o, int Hq, int Hkv,
    int max_length, int split_rows, int splits, float qk_scale,
    const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew,
    uint16_t *kw, uint16_t *vw, const int32_t *__restrict__ block_table,
    int max_blocks, int page_size, int num_pages, int head_major,
    const float *__restrict__ rcos, const float *__restrict__ rsin, int B,
    int P, int C_min, int hgs) {
  constexpr bool APPEND = MODE == 1 || MODE == 3;
  constexpr bool PAGED = MODE == 2;
  constexpr bool ROPE = MODE == 3;
  using T = Bf16Tile<D>;
  constexpr int BN = T::BN, KS = T::KS, NDB = T::NDB, NKB = T::NKB;
  constexpr int SV = T::SV;
  constexpr int LDS_MAIN = 4 * T::VT_BYTES;
  constexpr int LDS_FIN = (4 * G * D + 8 * 16) * 4;
  constexpr int LDS_BYTES = LDS_MAIN > LDS_FIN ? LDS_MAIN : LDS_FIN;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  __shared__ float fin_m[G], fin_l[G];
  // Each wave's K tile in LDS, 16-byte chunk c of row r
  // at chunk position c ^ kswz(r), so that the 16 rows of one A-operand read
  // fall on distinct banks. K is loaded as whole rows (four 256-byte rows per
  // instruction at D = 128, as V) rather than straight into the A-operand
  // layout (16 rows x 64 bytes per instruction): a compute-free read of the
  // two patterns streams 6.9 against 5.7 TB/s; the ragged batch of 64
  // sequences runs 156.6 against 159.7 us per call, 64 sequences at
  // position 4095 on the plain grid 171.0 against 177.2 us.
  __shared__ __attribute__((aligned(16))) unsigned char ksm[4 * BN * D * 2];
  // rotated new key (one per wave when the waves work alone)
  __shared__ __attribute__((aligned(16))) uint16_t krot[ROPE ? (SOLO ? 4 : 1) * D : 8];

  const int tid = threadIdx.x;
  // (uniform wave index in a scalar register where the paged tile lookup
  // depends on it)
  const int w = PAGED ? __builtin_amdgcn_readfirstlane(tid / 64) : tid / 64;
  const int l = tid % 64;
  const int li = l % 16;   // query column / row within a 16-row block
  const int lg = l / 16;   // lane group (k slots 8*lg..8*lg+7)
  const int oct = l % T::NOCT;  // V transpose item: rows 8*oct..8*oct+7
  const int ch = l / T::NOCT;   //                   dims 8*ch..8*ch+7
  uint16_t *vt = reinterpret_cast<uint16_t *>(smem + w * T::VT_BYTES);

  // Paged caches: row r of sequence b is row r % page_size of page
  // block_table[b][r / page_size] (clamped to the pages that exist), pages
  // token-major [page][row][Hkv][D] (consecutive rows of one kv head Hkv*D
  // elements apart) or head-major [page][Hkv][row][D] (rows of a head
  // contiguous). A tile (BN rows from a multiple of BN) never straddles a
  // page. (The lookup is made on wave-uniform values so that it is a scalar
  // load: a vector load would complete in order behind the K/V loads in
  // flight.)
  const size_t prs = head_major ? (size_t)D : (size_t)Hkv * D;
  auto page_of = [&](int bu, int t0) {
    const int tu = __builtin_amdgcn_readfirstlane(t0);
    const int pg = block_table[(size_t)bu * max_blocks + tu / page_size];
    return min(max(pg, 0), num_pages - 1);
  };
  auto page_tile = [&](const uint16_t *base, int gu, int pg, int t0) {
    const int tu = __builtin_amdgcn_readfirstlane(t0);
    return base + (head_major ? (((size_t)pg * Hkv + gu) * page_size + tu % page_size) * D
                              : ((size_t)pg * page_size + tu % page_size) * prs + (size_t)gu * D);
  };

  // Where the rows of a piece come from. Appending: the sequence's last valid
  // row (arow) is the new token; its K and V are read from knew / vnew, so no
  // workgroup reads that cache row while it is being written.
  struct Src {
    const uint16_t *kb, *vb, *kn, *vn;
    int b, g, last_row, arow;
  };
  auto src_of = [&](const Piece &p) {
    Src s;
    const size_t kvbase = ((size_t)p.b * Hkv + p.g) * (size_t)max_length * D;
    s.kb = kg + kvbase;
    s.vb = vg + kvbase;
    s.kn = knew + ((size_t)p.b * Hkv + p.g) * D;
    s.vn = vnew + ((size_t)p.b * Hkv + p.g) * D;
    s.b = p.b;
    s.g = p.g;
    s.last_row = p.row1 - 1;  // rows are clamped to the piece (masked later)
    s.arow = APPEND ? p.L - 1 : -1;
    return s;
  };

  u32x4_t kf[NKB][KS], vr[8], qv[KS];
  u32x4_t kraw[8];  // this wave's K tile as loaded: rows 8*oct + i, chunk ch
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  u32x4_t *kw_lds = reinterpret_cast<u32x4_t *>(ksm + w * BN * D * 2);
  bf16x8_t qf[KS];
  auto load_q = [&](const Piece &p) {
    const uint16_t *qrow = qg + ((size_t)p.b * Hq + (size_t)p.g * G + li) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks] = u32x4_t{0u, 0u, 0u, 0u};
      if (li < G) qv[ks] = *reinterpret_cast<const u32x4_t *>(qrow + ks * 32 + 8 * lg);
    }
  };
  auto load_k = [&](const Src &s, int t0, int pg) {
    const uint16_t *kt = PAGED ? page_tile(kg, s.g, pg, t0) : nullptr;
    // whole rows, as V: rows 8*oct + i, chunk ch
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(t0 + 8 * oct + i, s.last_row);
      const uint16_t *src = PAGED ? kt + (size_t)(row - t0) * prs
                                  : (APPEND && row == s.arow ? s.kn : s.kb + (size_t)row * D);
      kraw[i] = ldnt(src + 8 * ch);
    }
  };
  auto load_v = [&](const Src &s, int t0, int pg) {
    const uint16_t *vtl = PAGED ? page_tile(vg, s.g, pg, t0) : nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(t0 + 8 * oct + i, s.last_row);
      const uint16_t *src = PAGED ? vtl + (size_t)(row - t0) * prs
                                  : (APPEND && row == s.arow ? s.vn : s.vb + (size_t)row * D);
      vr[i] = ldnt(src + 8 * ch);
    }
  };
  // Runs piece `cur`. Each wave walks its tiles t0 = row0 + w*BN + 4*BN*i
  // (SOLO: all the piece's tiles, t0 = row0 + BN*i);
  // the next tile's K is loaded as soon as the score products have read the
  // current K registers and its V as soon as the current V rows are in LDS,
  // so both loads run during the softmax and P·V of this tile. (Loading the
  // first tile of the workgroup's next piece there as well, so that the
  // loads stay in flight through the merge of the four waves, was measured
  // 1-2 % slower on the ragged batch and batches of equal lengths.)
  auto run = [&](const Piece &cur_) __attribute__((always_inline)) {
  // (the piece is the same in every lane; held in scalar registers, the
  // addresses and loop bounds derived from it stay scalar too)
  Piece cur;
  cur.b = __builtin_amdgcn_readfirstlane(cur_.b);
  cur.g = __builtin_amdgcn_readfirstlane(cur_.g);
  cur.row0 = __builtin_amdgcn_readfirstlane(cur_.row0);
  cur.row1 = __builtin_amdgcn_readfirstlane(cur_.row1);
  cur.L = __builtin_amdgcn_readfirstlane(cur_.L);
  cur.slot = __builtin_amdgcn_readfirstlane(cur_.slot);
  cur.direct = __builtin_amdgcn_readfirstlane(cur_.direct);
  const int b = cur.b, g = cur.g, row0 = cur.row0, row1 = cur.row1;
  const Src cs = src_of(cur);
  constexpr int WS = SOLO ? 1 : 4;  // waves sharing the piece's tiles
  const int wofs = SOLO ? 0 : w;    // this wave's first tile of the piece
  uint16_t *kr = krot + (ROPE && SOLO ? w * D : 0);

  // Query heads of the group as the B operand of Sᵀ = K·Qᵀ (column li).
  // Rotary embedding: chunk ks of a lane (elements ks*32 + 8*lg ...) pairs
  // with chunk ks + KS/2 of the same lane (D/2 further on). (The rotation
  // waits for the tables; it is made after the first tile's loads are issued
  // so that their latency overlaps it.)
  load_q(cur);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(qv[ks]);
  auto rotate_q = [&]() {
    if (li < G) {
      const float *cb = rcos + (size_t)b * D, *sb = rsin + (size_t)b * D;
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        const int j0 = ks * 32 + 8 * lg;
        const u32x4_t lo = qv[ks], hi = qv[ks + KS / 2];
        qv[ks] = rope_bf16x8(lo, hi, cb + j0, sb + j0, true);
        qv[ks + KS / 2] = rope_bf16x8(hi, lo, cb + j0 + D / 2, sb + j0 + D / 2, false);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(qv[ks]);
  };

  // The piece that starts at row 0 stores the new token's K and V into the
  // cache. With the rotary embedding that piece and the piece that holds the
  // new row rotate the new key (into LDS, krot, for the latter); the wave
  // whose tile holds the new row takes that row's K from there.
  const int arow = cs.arow;
  const bool holds_arow = ROPE && row0 <= arow && arow < row1;  // uniform
  if (APPEND && (row0 == 0 || holds_arow)) {
    const size_t kvbase = ((size_t)b * Hkv + g) * (size_t)max_length * D;
    for (int i = SOLO ? l : tid; i < D / 8; i += SOLO ? 64 : kThreads) {
      u32x4_t kx = *reinterpret_cast<const u32x4_t *>(cs.kn + 8 * i);
      if constexpr (ROPE) {
        const int j0 = 8 * i;
        const bool lo = j0 < D / 2;
        const u32x4_t px = *reinterpret_cast<const u32x4_t *>(cs.kn + (lo ? j0 + D / 2 : j0 - D / 2));
        kx = rope_bf16x8(kx, px, rcos + (size_t)b * D + j0, rsin + (size_t)b * D + j0, lo);
        if (holds_arow) *reinterpret_cast<u32x4_t *>(&kr[j0]) = kx;
      }
      if (row0 == 0) {
        *reinterpret_cast<u32x4_t *>(kw + kvbase + (size_t)arow * D + 8 * i) = kx;
        *reinterpret_cast<u32x4_t *>(vw + kvbase + (size_t)arow * D + 8 * i) =
            *reinterpret_cast<const u32x4_t *>(cs.vn + 8 * i);
      }
    }
    if (holds_arow) {  // krot complete (uniform over the workgroup / wave)
      if constexpr (SOLO) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      } else {
        __syncthreads();
      }
    }
  }

  f32x4_t o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;
  float lsum = 0.f;

  // tnext >= 0: load that tile once this tile's registers are free
  auto compute_tile = [&](int t0, int tnext, int pgnext) {
    const bool full = t0 + BN <= row1;
    {
      // K rows -> the wave's LDS tile -> A operands; the next tile's rows
      // are requested as soon as these registers are written out
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * oct + i;
        kw_lds[r * CPR + (ch ^ kswz(r))] = kraw[i];
      }
      if (tnext >= 0) load_k(cs, tnext, pgnext);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int kb16 = 0; kb16 < NKB; ++kb16) {
        const int r = kb16 * 16 + li;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[kb16][ks] = kw_lds[r * CPR + ((4 * ks + lg) ^ kswz(r))];
      }
    }
    if constexpr (ROPE) {
      if (t0 <= arow && arow < t0 + BN) {  // this tile holds the new token
#pragma unroll
        for (int kb16 = 0; kb16 < NKB; ++kb16)
          if (t0 + kb16 * 16 + li == arow) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              kf[kb16][ks] = *reinterpret_cast<const u32x4_t *>(&kr[ks * 32 + 8 * lg]);
          }
      }
    }
    // ---- Sᵀ = K·Qᵀ --------------------------------------------------------------
    f32x4_t sc[NKB];
#pragma unroll
    for (int kb16 = 0; kb16 < NKB; ++kb16) {
      sc[kb16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[kb16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf[kb16][ks]), qf[ks], sc[kb16], 0, 0, 0);
    }
    // ---- V rows -> Vᵀ in LDS (keys 8*oct..8*oct+7 of dims 8*ch..8*ch+7) ----
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int wi = e / 2;
      u32x4_t pk;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t a = vr[2 * pr][wi], c = vr[2 * pr + 1][wi];
        pk[pr] = (e & 1) ? ((a >> 16) | (c & 0xffff0000u))
                         : ((a & 0xffffu) | (c << 16));
      }
      // rows of Vᵀ are 8-byte aligned (stride SV): two 8-byte writes
      u32x2_t *dst = reinterpret_cast<u32x2_t *>(&vt[(8 * ch + e) * SV + 8 * oct]);
      dst[0] = u32x2_t{pk[0], pk[1]};
      dst[1] = u32x2_t{pk[2], pk[3]};
    }
    if (tnext >= 0) load_v(cs, tnext, pgnext);
    // ---- online softmax -----------------------------------------------------------
    float mx = kNegInf;
#pragma unroll
    for (int kb16 = 0; kb16 < NKB; ++kb16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[kb16][r] * qk_scale;
        if (!full && t0 + kb16 * 16 + 4 * lg + r >= row1) x = kNegInf;
        sc[kb16][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);  // finite: the tile's first row is valid
    if (__any(mnew > m)) {
      const float alpha = fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m = mnew;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- Oᵀ += Vᵀ·Pᵀ ---------------------------------------------------------------
#pragma unroll
    for (int t2 = 0; t2 < BN / 32; ++t2) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(sc[2 * t2][r] - m);
        p[4 + r] = fast_exp2(sc[2 * t2 + 1][r] - m);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lsum += p[e];
      const u32x4_t pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      const bf16x8_t pb = as_bf16x8(pw);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t *vrow = &vt[(db * 16 + li) * SV + 32 * t2 + 4 * lg];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + 16);
        const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), pb,
                                                       o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int t0 = row0 + wofs * BN, first = 1; t0 < row1; t0 += WS * BN, first = 0) {
    if (first) {
      const int pg0 = PAGED ? page_of(b, t0) : 0;
      load_k(cs, t0, pg0);
      load_v(cs, t0, pg0);
      if constexpr (ROPE) rotate_q();
    }
    const int t1 = t0 + WS * BN;
    // (the next tile's page is looked up before this tile's products, so the
    // scalar load has completed when the next tile's loads are issued)
    const int pg1 = PAGED && t1 < row1 ? page_of(b, t1) : 0;
    compute_tile(t0, t1 < row1 ? t1 : -1, pg1);
  }

  lsum += __shfl_xor(lsum, 16);  // the four lane groups of a query
  lsum += __shfl_xor(lsum, 32);
  if constexpr (SOLO) {
    // The wave's own result for the G query heads: lane (li < G, lg) holds
    // output dimensions db*16 + 4*lg + r of query head li.
    if (li < G) {
      const size_t head = (size_t)b * Hq + (size_t)g * G + li;
      if (cur.direct) {  // (divided as the merged form divides)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          uint32_t *dst = static_cast<uint32_t *>(outp) + (head * D + db * 16 + 4 * lg) / 2;
          *reinterpret_cast<u32x2_t *>(dst) =
              u32x2_t{pack_bf16x2(o[db][0] / lsum, o[db][1] / lsum),
                      pack_bf16x2(o[db][2] / lsum, o[db][3] / lsum)};
        }
      } else {
        const size_t ps = head * splits + cur.slot;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4_t *>(ws_o + ps * D + db * 16 + 4 * lg) = o[db];
        if (lg == 0) *reinterpret_cast<float2 *>(ws_ml + ps * 2) = make_float2(m, lsum);
      }
    }
    return;
  } else {
  // ---- merge the 4 waves -----------------------------------------------------------
  __syncthreads();  // every wave is done with its Vᵀ tile
  float *wm = reinterpret_cast<float *>(smem);  // [4][16]
  float *wl = wm + 4 * 16;                      // [4][16]
  float *wo = wl + 4 * 16;                      // [4][G][D]
  if (lg == 0) {
    wm[w * 16 + li] = m;
    wl[w * 16 + li] = lsum;
  }
  if (li < G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4_t *>(&wo[(w * G + li) * D + db * 16 + 4 * lg]) = o[db];
  }
  __syncthreads();
  float *fo = wo;  // merged output overwrites wave 0's slot, read first
  if (tid < G) {
    float x = wm[tid];
    for (int i = 1; i < 4; ++i) x = fmaxf(x, wm[i * 16 + tid]);
    float lt = 0.f;
    for (int i = 0; i < 4; ++i) lt += fast_exp2(wm[i * 16 + tid] - x) * wl[i * 16 + tid];
    fin_m[tid] = x;
    fin_l[tid] = lt;
  }
  __syncthreads();
  float acc[(G * D + kThreads - 1) / kThreads];
#pragma unroll
  for (int j = 0; j * kThreads < G * D; ++j) {
    const int i = tid + j * kThreads;
    acc[j] = 0.f;
    if (i < G * D) {
      const int h = i / D;
      const float mh = fin_m[h];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        acc[j] = fmaf(fast_exp2(wm[ww * 16 + h] - mh), wo[ww * G * D + i], acc[j]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j * kThreads < G * D; ++j) {
    const int i = tid + j * kThreads;
    if (i < G * D) fo[i] = acc[j];
  }
  __syncthreads();
  finish<true, D, G, kThreads>(fin_m, fin_l, fo, cur.direct != 0, b, g, cur.slot, Hq,
                               splits, outp, ws_ml, ws_o);
  }  // !SOLO
  };  // run

  if constexpr (SOLO) {
    // Worker u takes the tiles [u*C, min((u+1)*C, TT)) of the batch's
    // (b, h, tile) order (balanced schedule). hgs == 1: h is the kv head and
    // every wave a worker, u = 4 * wg + w, P workers. hgs == 4 (Hkv a multiple
    // of 4): h is a group of four kv heads and every workgroup a worker,
    // u = wg, P / 4 workers; its wave w takes kv head 4h + w of every tile,
    // so that the four waves read neighbouring slices of the same token rows.
    // Workgroup i runs on XCD i % 8: wg = (i % 8) * (P / 32) + i / 8 gives
    // each XCD a contiguous run of workers (P / 4 is a multiple of 8).
    const int NH = Hkv / hgs;  // units h per sequence
    const BatchTiles bt = batch_tiles(seq_lens, B, max_length, BN);
    const int TT = NH * bt.total;
    const int C = chunk_tiles(TT, hgs == 1 ? P : P / 4, C_min);
    const int wg = (int)(blockIdx.x % 8) * (P / 32) + (int)blockIdx.x / 8;
    const int u = hgs == 1 ? 4 * wg + w : wg;
    const int lo = u * C;
    if (lo >= TT) return;  // (no workgroup barrier follows in this path)
    const int hi = min(lo + C, TT);
    // the sequence of tile lo: the first b with NH * (tiles up to b) > lo
    int b = 0;
#pragma unroll
    for (int c = 0; c < kBalancedMaxB / 64; ++c) {
      const unsigned long long hit = __ballot(NH * bt.incl[c] > lo);
      if (hit != 0ull) {
        b = 64 * c + __ffsll(hit) - 1;
        break;
      }
    }
    b = __builtin_amdgcn_readfirstlane(b);
    int nb = seq_value(bt.cnt, b);
    int Pb = seq_value(bt.incl, b) - nb;
    int Lb = seq_value(bt.len, b);
    int h = (lo - NH * Pb) / nb;
    // the piece of (b, h) from tile `from` up to the range's end; its end tile
    auto piece_at = [&](int from, int &end) {
      const int start = NH * Pb + h * nb;   // first tile of (b, h)
      const int t_end = min(nb, hi - start);
      const int first = start / C;          // worker holding tile 0 of (b, h)
      Piece p;
      p.b = b;
      p.g = hgs == 1 ? h : hgs * h + w;
      p.row0 = (from - start) * BN;
      p.row1 = min(t_end * BN, Lb);
      p.L = Lb;
      p.slot = u - first;
      p.direct = first == (start + nb - 1) / C;
      end = start + t_end;
      return p;
    };
    int from = lo, end;
    for (;;) {
      run(piece_at(from, end));
      if (end >= hi) break;
      // the next piece is tile 0 of the next (b, h)
      if (++h == NH) {  // next sequence that holds rows
        h = 0;
        Pb += nb;
        nb = 0;
        while (nb == 0 && b + 1 < B) {
          ++b;
          Lb = seq_value(bt.len, b);
          nb = (Lb + BN - 1) / BN;
        }
        if (nb == 0) break;  // (not reached: tiles remain, so rows do)
      }
      from = end;
    }
  } else {
  const Unit un = locate_unit(seq_lens, gridDim.y, Hkv, max_length, split_rows);
  if (un.b < 0) return;
  const Item it = make_item(seq_lens, un.b, position_id, max_length, split_rows, un.s);
  if (it.row0 >= it.L) {
    if (it.L == 0 && un.s == 0) write_zero_rows<true, D, G, kThreads>(outp, un.b, un.g, Hq);
    return;
  }
  run(Piece{un.b, un.g, it.row0, it.row1, it.L, un.s, it.n_split == 1});
  }  // !SOLO
}

// ---------------------------------------------------------------------------
// fp32: vector-ALU form
// ---------------------------------------------------------------------------
template <int D, int G, bool APPEND, bool ROPE>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp,
    const float *__restrict__ vp, const int32_t *__restrict__ seq_lens,
    int position_id, void *__restrict__ outp, float *__restrict__ ws_ml,
    float *__restrict__ ws_o, int Hq, int Hkv,
    int max_length, int split_rows, int splits, float qscale,
    const float *__restrict__ knew, const float *__restrict__ vnew,
    float *kw, float *vw, const float *__restrict__ rcos,
    const float *__restrict__ rsin) {
  constexpr int VEC = 4;                // floats per 16-byte chunk
  constexpr int LPR = D / VEC;          // lanes per cache row (16 or 32)
  constexpr int NG = kThreads / LPR;    // row groups per workgroup
  constexpr int U = 4;                  // rows per group per iteration
  __shared__ float sm_m[NG][G];
  __shared__ float sm_l[NG][G];
  __shared__ float sm_o[G * D];
  __shared__ float fin_m[G], fin_l[G];

  const Unit un = locate_unit(seq_lens, gridDim.y, Hkv, max_length, split_rows);
  if (un.b < 0) return;
  const int g = un.g, b = un.b, s = un.s;
  const Item it = make_item(seq_lens, b, position_id, max_length, split_rows, s);
  if (it.row0 >= it.L) {
    if (it.L == 0 && s == 0) write_zero_rows<false, D, G, kThreads>(outp, b, g, Hq);
    return;
  }
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int grp = tid / LPR;

  // Rotary embedding: lane lr's elements pair with those of lane lr ± LPR/2
  // (D/2 away), read again from memory.
  const bool rlo = lr < LPR / 2;
  const int rpart = (lr * VEC + D / 2) % D;
  float qv[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float *qrow = qp + ((size_t)b * Hq + (size_t)g * G + h) * D;
    u32x4_t x = *reinterpret_cast<const u32x4_t *>(qrow + lr * VEC);
    if constexpr (ROPE)
      x = rope_f32x4(x, *reinterpret_cast<const u32x4_t *>(qrow + rpart),
                     rcos + (size_t)b * D + lr * VEC, rsin + (size_t)b * D + lr * VEC, rlo);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[h][e] = __uint_as_float(x[e]) * qscale;
  }
  float m[G], l[G], o[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
  }
  const size_t rowbase = ((size_t)b * Hkv + g) * (size_t)max_length;
  const float *kb = kp + rowbase * D + lr * VEC;
  const float *vb = vp + rowbase * D + lr * VEC;
  // Appending: as in the bf16 kernel, the last valid row is read from knew /
  // vnew and split 0 stores it into the cache; with the rotary embedding the
  // rotated key chunk is kept in registers (knr).
  const int arow = APPEND ? it.L - 1 : -1;
  const float *kn = knew + ((size_t)b * Hkv + g) * D + lr * VEC;
  const float *vn = vnew + ((size_t)b * Hkv + g) * D + lr * VEC;
  u32x4_t knr = {0u, 0u, 0u, 0u};
  if constexpr (ROPE)
    knr = rope_f32x4(*reinterpret_cast<const u32x4_t *>(kn),
                     *reinterpret_cast<const u32x4_t *>(knew + ((size_t)b * Hkv + g) * D + rpart),
                     rcos + (size_t)b * D + lr * VEC, rsin + (size_t)b * D + lr * VEC, rlo);
  if (APPEND && s == 0 && tid < LPR) {
    *reinterpret_cast<u32x4_t *>(kw + (rowbase + arow) * D + lr * VEC) =
        ROPE ? knr : *reinterpret_cast<const u32x4_t *>(kn);
    *reinterpret_cast<u32x4_t *>(vw + (rowbase + arow) * D + lr * VEC) =
        *reinterpret_cast<const u32x4_t *>(vn);
  }

  for (int r = it.row0 + grp; r < it.row1; r += NG * U) {
    u32x4_t kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + u * NG;
      kr[u] = u32x4_t{0u, 0u, 0u, 0u};
      vr[u] = kr[u];
      if (rr < it.row1) {
        if (ROPE && rr == arow)
          kr[u] = knr;
        else
          kr[u] = ldnt(APPEND && rr == arow ? kn : kb + (size_t)rr * D);
        vr[u] = ldnt(APPEND && rr == arow ? vn : vb + (size_t)rr * D);
      }
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(qv[h][e], __uint_as_float(kr[u][e]), acc);
        sc[u][h] = group_sum<LPR>(acc);
      }
      if (r + u * NG >= it.row1) {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[u][h] = kNegInf;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
      const float mnew = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - mnew);
      float p[U];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = fast_exp2(sc[u][h] - mnew);
        ps += p[u];
      }
      l[h] = fmaf(l[h], alpha, ps);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = o[h][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fmaf(p[u], __uint_as_float(vr[u][e]), acc);
        o[h][e] = acc;
      }
      m[h] = mnew;
    }
  }

  // merge the row groups: common max, rescale, sum (fixed order)
  if (lr == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[grp][h] = m[h];
      sm_l[grp][h] = l[h];
    }
  }
  __syncthreads();
  if (tid < G) {
    float x = sm_m[0][tid];
    for (int i = 1; i < NG; ++i) x = fmaxf(x, sm_m[i][tid]);
    float lt = 0.f;
    for (int i = 0; i < NG; ++i) lt += fast_exp2(sm_m[i][tid] - x) * sm_l[i][tid];
    fin_m[tid] = x;
    fin_l[tid] = lt;
  }
  for (int i = tid; i < G * D; i += kThreads) sm_o[i] = 0.f;
  __syncthreads();
  float w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) w[h] = fast_exp2(m[h] - fin_m[h]);
  // groups add their rescaled output one at a time (deterministic order)
  for (int i = 0; i < NG; ++i) {
    if (grp == i) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_o[h * D + lr * VEC + e] += w[h] * o[h][e];
    }
    __syncthreads();
  }
  finish<false, D, G, kThreads>(fin_m, fin_l, sm_o, it.n_split == 1, b, g, s,
                                Hq, splits, outp, ws_ml, ws_o);
}

// ---------------------------------------------------------------------------
// Combine: one workgroup per (kv head, sequence) with more than one split;
// wave h merges query head g*G+h. Lane t takes the (max, sum) of splits
// t, t+64, ...; the wave reduces the global max, the weights 2^(m_s - M)
// go to LDS, and every lane then sums its output dimensions over the splits
// in split order with independent (unrolled) loads.
// ---------------------------------------------------------------------------

// One wave per (query head, sequence). The loads of the first 64 partial
// outputs are issued before the running maxima and sums are read, so a
// sequence with up to 64 splits is merged after a single memory round trip;
// further chunks of 64 follow one round trip each. Lane l holds output
// dimensions [l*D/64, (l+1)*D/64); the weight of split t sits in lane t % 64
// of its chunk and is broadcast with a lane read.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float *__restrict__ ws_ml, const float *__restrict__ ws_o,
    const int32_t *__restrict__ seq_lens, int position_id,
    void *__restrict__ outp, int Hq, int max_length, int split_rows,
    int splits, int Hkv, int balanced, int P, int C_min, int hgs) {
  constexpr int PER = D / 64;  // output dimensions per lane
  static_assert(PER == 1 || PER == 2, "D is 64 or 128");
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const size_t head = (size_t)b * Hq + hq;
  int n;  // partials of (b, hq)
  if (balanced) {
    // the pieces of (b, g) under the balanced schedule (above); a sequence
    // without rows gets its zero output row here
    constexpr int BN = 4096 / D;
    const BatchTiles bt = batch_tiles(seq_lens, gridDim.y, max_length, BN);
    const int nb = seq_value(bt.cnt, b);
    const int Pb = seq_value(bt.incl, b) - nb;
    if (nb == 0) {
#pragma unroll
      for (int e = 0; e < PER; ++e) store_out<BF16>(outp, head * D + lane * PER + e, 0.f);
      return;
    }
    const int NH = Hkv / hgs;  // units per sequence
    const int C = chunk_tiles(NH * bt.total, hgs == 1 ? P : P / 4, C_min);
    const int start = NH * Pb + (hq / (Hq / Hkv)) / hgs * nb;
    n = (start + nb - 1) / C - start / C + 1;
  } else {
    n = make_item(seq_lens, b, position_id, max_length, split_rows, 0).n_split;
  }
  if (n <= 1) return;  // finished by the split kernel (or zero rows)
  const float2 *ml = reinterpret_cast<const float2 *>(ws_ml + head * splits * 2);
  const float *o = ws_o + head * splits * D + lane * PER;
  const int last = n - 1;
  // Partials t >= n are never written: their loads are clamped to split n-1
  // (finite) and their weight is 0.
  float v[64][PER];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (c0 + 16 * q < n) {
#pragma unroll
        for (int u = 16 * q; u < 16 * q + 16; ++u) {
          const float *src = o + (size_t)min(c0 + u, last) * D;
          if constexpr (PER == 2) {
            const float2 x = *reinterpret_cast<const float2 *>(src);
            v[u][0] = x.x;
            v[u][1] = x.y;
          } else {
            v[u][0] = src[0];
          }
        }
      }
    }
  };
  load_chunk(0);
  const float2 ml0 = ml[min(lane, last)];
  float mx = ml0.x;
  for (int t = lane + 64; t < n; t += 64) mx = fmaxf(mx, ml[t].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float wl = lane < n ? fast_exp2(ml0.x - mx) : 0.f;
  float lt = wl * ml0.y;
  for (int t = lane + 64; t < n; t += 64) {
    const float2 x = ml[t];
    lt = fmaf(fast_exp2(x.x - mx), x.y, lt);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c0 = 0;;) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (c0 + 16 * q < n) {
#pragma unroll
        for (int u = 16 * q; u < 16 * q + 16; ++u) {
          const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] = fmaf(wt, v[u][e], acc[e]);
        }
      }
    }
    c0 += 64;
    if (c0 >= n) break;
    load_chunk(c0);
    const int t = c0 + lane;
    wl = t < n ? fast_exp2(ml[min(t, last)].x - mx) : 0.f;
  }
  const float inv = 1.f / lt;
  const size_t oi = head * D + lane * PER;
  if constexpr (PER == 2) {
    if constexpr (BF16) {
      static_cast<uint32_t *>(outp)[oi / 2] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      *reinterpret_cast<float2 *>(static_cast<float *>(outp) + oi) =
          make_float2(acc[0] * inv, acc[1] * inv);
    }
  } else {
    store_out<BF16>(outp, oi, acc[0] * inv);
  }
}


template <bool BF16, int D, int G, int MODE>
void launch_split(const DecodeArgs &a, hipStream_t stream) {
  // (balanced: P workers, four per workgroup)
  const dim3 grid = a.plan.balanced ? dim3(a.plan.P / 4) : dim3(a.Hkv, a.B, a.plan.splits);
  if constexpr (BF16) {
    auto *kern = a.plan.balanced ? decode_bf16_kernel<D, G, MODE, true>
                                 : decode_bf16_kernel<D, G, MODE, false>;
    kern<<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
        static_cast<const uint16_t *>(a.v), a.seq_lens, a.position_id, a.out,
        a.ws_ml, a.ws_o, a.Hq, a.Hkv, a.max_length,
        a.plan.split_rows, a.plan.splits, a.scale * kLog2e,
        static_cast<const uint16_t *>(a.k_new), static_cast<const uint16_t *>(a.v_new),
        static_cast<uint16_t *>(a.k_w), static_cast<uint16_t *>(a.v_w),
        a.block_table, a.max_blocks, a.page_size, a.num_pages, a.head_major,
        a.rope_cos, a.rope_sin, a.B, a.plan.P, a.plan.C_min, a.plan.hgs);
  } else {
    static_assert(MODE != 2, "paged caches are bf16 only");
    decode_f32_kernel<D, G, MODE == 1 || MODE == 3, MODE == 3><<<grid, kThreads, 0, stream>>>(
        static_cast<const float *>(a.q), static_cast<const float *>(a.k),
        static_cast<const float *>(a.v), a.seq_lens, a.position_id, a.out,
        a.ws_ml, a.ws_o, a.Hq, a.Hkv, a.max_length,
        a.plan.split_rows, a.plan.splits, a.scale * kLog2e,
        static_cast<const float *>(a.k_new), static_cast<const float *>(a.v_new),
        static_cast<float *>(a.k_w), static_cast<float *>(a.v_w), a.rope_cos,
        a.rope_sin);
  }
}

template <bool BF16, int D, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
  if (a.k_new != nullptr && a.rope_cos != nullptr)
    launch_split<BF16, D, G, 3>(a, stream);
  else if (a.k_new != nullptr)
    launch_split<BF16, D, G, 1>(a, stream);
  else if constexpr (BF16) {
    if (a.block_table != nullptr)
      launch_split<BF16, D, G, 2>(a, stream);
    else
      launch_split<BF16, D, G, 0>(a, stream);
  } else {
    launch_split<BF16, D, G, 0>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!a.plan.balanced && a.plan.splits <= 1)) return e;
  decode_combine_kernel<BF16, D><<<dim3(a.Hq, a.B), 64, 0, stream>>>(
      a.ws_ml, a.ws_o, a.seq_lens, a.position_id, a.out, a.Hq, a.max_length,
      a.plan.split_rows, a.plan.splits, a.Hkv, a.plan.balanced, a.plan.P,
      a.plan.C_min, a.plan.hgs);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_typed<BF16, D, 1>(a, stream);
    case 2: return launch_typed<BF16, D, 2>(a, stream);
    case 4: return launch_typed<BF16, D, 4>(a, stream);
    case 8: return launch_typed<BF16, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.bf16) {
    return a.D == 64 ? launch_d<true, 64>(a, stream)
                     : launch_d<true, 128>(a, stream);
  }
  return a.D == 64 ? launch_d<false, 64>(a, stream)
                   : launch_d<false, 128>(a, stream);
}

}  // namespace attn
