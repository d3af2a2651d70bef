// Causal prefill against a cached prefix on bf16 matrix cores (gfx950).
//
// Operation: "step14_3 — batched attention: removing the per-head Python
// loop", solution section — for every head at once, scores = Q·Kᵀ scaled by
// 1/sqrt(d_head), causal entries set to -inf, softmax over each row, times V;
// the going-further section fuses the three steps into one kernel so the
// score matrix never reaches HBM. New token i sits at cache row prefix+i and
// sees rows [0, prefix+i].
//
// One kernel for D = 64 and D = 128 (prefill_lds_kernel): one workgroup =
// 8 waves = 64 queries of one head, walking the key tiles (8 KiB of K each:
// 64 keys at D = 64, 32 at D = 128) up to the causal bound of its last query.
//   * Waves: query group qg = w / 4 (32 queries, two 16-column blocks: every
//     K and V operand feeds two products) x key quarter kq = w % 4 (tiles t
//     with t % 4 == kq). Two waves per SIMD. The four key quarters of a query
//     group are merged (log-sum-exp) in LDS at the end.
//   * Block -> work map: workgroup id i runs on XCD i % 8; each XCD takes a
//     contiguous run of head instances, so every query tile of a head, and
//     every query head of a kv head (grouped-query attention), reads that kv
//     head's K and V through the same L2, fetched from HBM about once; on
//     each XCD tiles run longest first.
//   * Each iteration's four K tiles and four V tiles cross the L1 path once
//     per workgroup, as buffer loads that write LDS directly, double-buffered,
//     one workgroup barrier per iteration; the next iteration's loads are
//     issued before the current one is computed.
//   * Sᵀ = K·Qᵀ on v_mfma_f32_16x16x32_bf16 (A = 16 key rows from LDS, B =
//     the wave's queries in registers) puts each lane on one query and 4 keys
//     of every 16-key block: the operand layout of Oᵀ += Vᵀ·Pᵀ, so P never
//     leaves registers; the Vᵀ operand comes from transposing LDS reads
//     (ds_read_b64_tr_b16).
//   * Softmax in the exp2 domain: each probability is one fma (fp32 score
//     times scale·log2 e, minus the running max) and one v_exp_f32; the
//     output is rescaled only when the running max grows by more than 8
//     (log2 units). Row sums come from the matrix cores: an
//     all-ones A operand times Pᵀ sums the same bf16 probabilities the output
//     uses.
//   * Only tiles that cross the diagonal evaluate the mask; tiles past a
//     query group's last visible key are skipped.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int NQG = 2;   // query groups per workgroup
constexpr int kXcds = 8;
constexpr int kCUs = 256;  // compute units of an MI355X
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag
// buffer resource word 3 for raw (untyped, stride 0) 32-bit accesses
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// max of three fp32 values in one v_max3_f32 (no operand quieting: the
// kernel's scores are never NaN).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ds_read_b64_tr_b16: in each group of 16 lanes, the 16 addresses name 16
// runs of 4 bf16 values M[s][0..3]; lane i receives M[i/4 + 4e][i%4] for
// e = 0..3 (a 4x4-blocked transpose).
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
__device__ __forceinline__ u32x2_t read_tr16(const uint16_t *lds) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t *)(const_cast<uint16_t *>(lds)));
  return __builtin_bit_cast(u32x2_t, r);
}

// ---------------------------------------------------------------------------
// K and V staged once per workgroup in LDS
// ---------------------------------------------------------------------------
//   * LDS tiles are unpadded rows of 2 D bytes; the 16-byte chunk c of row r
//     sits at c ^ swz_k(r) for K (the 16 rows x 16 bytes of one A-operand
//     read fall on distinct banks) and c ^ swz_v(r) for V (the 16 rows x 32
//     bytes of one transposing read spread evenly over the banks).
//   * K and V are read through buffer resources limited to the rows
//     [0, prefix + Lq): rows past the end read as zeros.
//   * The running max is reduced across the four lanes of a query with
//     v_permlane16_swap / v_permlane32_swap.
typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte-per-lane direct-to-LDS buffer load (1 KiB per wave at dst).
// (A plain function: called with template-dependent arguments straight from
// a kernel template, the builtin made the host pass drop the kernel's launch
// stub without a diagnostic.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst,
                                      int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}

// BN_: keys per tile. 4096 / D makes 8 KiB tiles; with NKQ_ = 4 key parts
// (waves per query group) one workgroup takes 130 KiB of LDS, one per CU.
// For grids with at least two workgroups per CU, 4 KiB tiles at D = 64, or
// two key parts at D = 128, halve that, so that two workgroups share a CU
// out of step with each other.
template <int D_, int BN_ = 4096 / D_, int NKQ_ = 4>
struct PT {
  static constexpr int D = D_, NB = 2, NQW = 16 * NB, BM = NQG * NQW;
  static constexpr int NKQ = NKQ_;
  static constexpr int THREADS = 64 * NQG * NKQ;
  static constexpr int BN = BN_;
  static constexpr int KS = D / 32, NDB = D / 16, NKB = BN / 16;
  static constexpr int ROWB = D * 2;             // bytes per cache row
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int RPL = 1024 / ROWB;        // rows per 1 KiB LDS load
  static constexpr int T_BYTES = BN * ROWB;      // one tile: 8 KiB
  static constexpr int DMA = T_BYTES / 1024;     // 1 KiB LDS loads per tile
  static constexpr int BUF = NKQ * T_BYTES;      // one iteration of K (or V)
  static constexpr int NPAR = D == 64 ? 2 : 4;   // distinct swizzles per load
  static_assert(BN % 32 == 0 && T_BYTES % 1024 == 0, "32-key steps, whole 1 KiB loads");
  // LDS position of 16-byte chunk c of tile row r. K: the 16 rows x 16
  // bytes of one A-operand read fall on distinct banks; V: the 16 rows x 32
  // bytes of one transposing read spread evenly over the banks.
  static __device__ __forceinline__ int swz_k(int r) {
    return D == 64 ? (r >> 1) & 7 : r & 15;
  }
  static __device__ __forceinline__ int swz_v(int r) {
    return D == 64 ? 2 * ((r >> 1) & 3) : 2 * (r & 7);
  }
};
using P64 = PT<64>;

__device__ __forceinline__ float quad_max(float m) {
  // max over lanes l, l ^ 16, l ^ 32, l ^ 48
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// PAGED: K and V rows come from pages of page_size rows (a multiple of the
// tile, so a tile never straddles pages) named by
// block_table[b][row / page_size] (clamped to the pages that exist); pages
// are token-major [page][row][Hkv][D] or head-major [page][Hkv][row][D].
template <int D_, bool PAGED, int BN_, int NKQ_>
__global__ __launch_bounds__(P64::THREADS) void prefill_lds_kernel(
    const uint16_t *__restrict__ qg, const uint16_t *__restrict__ kg,
    const uint16_t *__restrict__ vg, uint16_t *__restrict__ outg, int NH,
    int Hq, int Hkv, int max_length, int Lq, int prefix, float qk_scale,
    int n_qtiles, int heads_per_xcd, const int32_t *__restrict__ block_table,
    int max_blocks, int page_size, int num_pages, int head_major) {
  using T = PT<D_, BN_, NKQ_>;
  constexpr int NKQ = T::NKQ;
  constexpr int D = T::D, KS = T::KS, NDB = T::NDB, NKB = T::NKB, BN = T::BN;
  constexpr int NB = T::NB, NQW = T::NQW, BM = T::BM, ROWB = T::ROWB;
  // K and V buffers of the two iterations in flight, as separate LDS
  // objects: the compiler then tells a direct load into one from reads of
  // another and does not make the reads wait for it.
  __shared__ __attribute__((aligned(16))) unsigned char kb0[T::BUF], kb1[T::BUF],
      vb0[T::BUF], vb1[T::BUF];
  __shared__ float mml[2 * NQG * NQW * NKQ];  // merge: running max and sum

  // ---- work item: (head instance, query tile) -----------------------------------
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int k = id / kXcds;
  // XCD x takes head instances [x * heads_per_xcd, (x + 1) * heads_per_xcd):
  // consecutive query heads share a kv head, so a kv head's K and V are
  // fetched into one L2 for all the query heads that read them
  const int j = xcd * heads_per_xcd + k % heads_per_xcd;  // head instance b*Hq + h
  if (j >= NH) return;
  // (integer division runs on the vector ALUs; readfirstlane keeps the
  // workgroup-uniform results in scalar registers)
  const int qt = __builtin_amdgcn_readfirstlane(n_qtiles - 1 - k / heads_per_xcd);
  const int b = __builtin_amdgcn_readfirstlane(j / Hq);
  const int h = j % Hq;
  const int kvh = __builtin_amdgcn_readfirstlane(h / (Hq / Hkv));

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int l = tid % 64;
  const int li = l % 16;
  const int lg = l / 16;
  const int kq = w % NKQ;   // key quarter
  const int qgi = w / NKQ;  // query group

  const int kv_len = prefix + Lq;
  const int q_end = min((qt + 1) * BM, Lq);
  const int n_tiles = (prefix + q_end + BN - 1) / BN;  // tiles the workgroup sees
  const int n_iter = (n_tiles + NKQ - 1) / NKQ;
  const int qg0 = qt * BM + qgi * NQW;  // first query of this wave's group
  const bool g_active = qg0 < Lq;
  const int g_kmax = prefix + min(qg0 + NQW - 1, Lq - 1);  // last visible key

  const size_t kvbase = PAGED ? 0 : ((size_t)b * Hkv + kvh) * (size_t)max_length * D;
  // wave (0, kq) streams K, wave (1, kq) streams V
  const uint16_t *kvsrc = qgi == 0 ? kg : vg;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(kvsrc + kvbase), (short)0, kv_len * ROWB, kBufferFlags);
  // bytes between consecutive rows of one kv head (paged token-major pages
  // interleave the heads)
  const int prs = PAGED && !head_major ? Hkv * ROWB : ROWB;

  // This wave's queries as B operands (column li of block nb), as stored:
  // the scale is applied to the fp32 scores (folding it into bf16 queries
  // would add a relative error of 2^-9 to every score, which large scores
  // turn into visible weight errors).
  bf16x8_t qf[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qme = qg0 + nb * 16 + li;
    const size_t qrow = ((size_t)j * Lq + (size_t)qme) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qme < Lq) v = *reinterpret_cast<const u32x4_t *>(qg + qrow + ks * 32 + 8 * lg);
      qf[nb][ks] = as_bf16x8(v);
    }
  }
  const u32x4_t ones_w = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8_t ones = as_bf16x8(ones_w);

  f32x4_t o[NB][NDB];
  f32x4_t lacc[NB];
  float mc[NB];   // running max (log2 units), -inf before the first key
  float nmc[NB];  // exponent offset: -mc, 0 while mc = -inf
  float thr[NB];  // raw score above which the max must move: (mc + slack) / scale
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[nb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lacc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mc[nb] = kNegInf;
    nmc[nb] = 0.f;
    thr[nb] = kNegInf;
  }

  // Loads: load jj of a tile fills LDS bytes [1024 jj, 1024 jj + 1024); lane
  // l writes position l % CPR of row RPL jj + l / CPR and reads the chunk
  // that belongs there (the swizzles repeat every RPL * NPAR rows).
  int dma_off[T::NPAR];
#pragma unroll
  for (int par = 0; par < T::NPAR; ++par) {
    const int pos = l % T::CPR;
    const int r = T::RPL * par + l / T::CPR;
    const int chunk = pos ^ (qgi == 0 ? T::swz_k(r) : T::swz_v(r));
    dma_off[par] = (l / T::CPR) * prs + chunk * 16;
  }
  // Paged: element offset of the first row of tile t (rows r0 .. r0+BN-1 of
  // this kv head) in the page pool.
  auto tile_offset = [&](int t) -> uint64_t {
    const int r0 = t * BN;
    const int bi = min(r0 / page_size, max_blocks - 1);
    const int pg = min(max(block_table[(size_t)b * max_blocks + bi], 0), num_pages - 1);
    const int rin = r0 % page_size;
    return head_major ? (((uint64_t)pg * Hkv + kvh) * page_size + rin) * D
                      : ((uint64_t)pg * page_size + rin) * Hkv * D + (uint64_t)kvh * D;
  };
  // Lane i holds (in two halves) the offset of this wave's tile of
  // iteration i: one lookup per lane here, none before the issues.
  uint32_t po_lo = 0, po_hi = 0;
  if constexpr (PAGED) {
    const uint64_t off = tile_offset(l * NKQ + kq);
    po_lo = (uint32_t)off;
    po_hi = (uint32_t)(off >> 32);
  }
  auto issue = [&](int it, unsigned char *kbuf, unsigned char *vbuf) {
    unsigned char *dst = (qgi == 0 ? kbuf : vbuf) + kq * T::T_BYTES;
    const int t = it * NKQ + kq;
    if constexpr (PAGED) {
      // the tile's rows in the pool (lane `it` of po_lo/po_hi for the first
      // 64 iterations, else looked up: b, kq and it are wave-uniform) and a
      // resource over the rows that exist: rows past kv_len read as zeros
      uint64_t off;
      if (it < 64)
        off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)po_hi, it) << 32) |
              (uint32_t)__builtin_amdgcn_readlane((int)po_lo, it);
      else
        off = tile_offset(t);
      // (readfirstlane: the resource must sit in scalar registers; a clamp
      // computed on the vector ALUs would otherwise turn every load into a
      // loop over distinct resource values)
      const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(BN, kv_len - t * BN)) * prs);
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(kvsrc + off), (short)0, nbytes, kBufferFlags);
#pragma unroll
      for (int jj = 0; jj < T::DMA; ++jj)
        dma16(rt, dst + jj * 1024, dma_off[jj % T::NPAR], jj * T::RPL * prs);
    } else {
#pragma unroll
      for (int jj = 0; jj < T::DMA; ++jj)
        dma16(rs, dst + jj * 1024, dma_off[jj % T::NPAR], t * T::T_BYTES + jj * 1024);
    }
  };
  // A-operand reads of K: block kb, k-step ks -> row 16 kb + li, chunk
  // 4 ks + lg at position (4 ks + lg) ^ swz_k(li) (swz_k has period 16).
  int kro[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kro[ks] = li * ROWB + (((4 * ks + lg) ^ T::swz_k(li)) * 16);
  // Transposing reads of V: lane (li, lg) names row r = 4 lg + li / 4 (+ 32
  // t2, + 16: swz_v has period 8) and the 8 bytes of chunk 2 db + (li >> 1)
  // % 2, half li % 2; swz_v is even, so the chunk pair 2 db, 2 db + 1 moves
  // as a unit to position pair 2 (db ^ swz_v(r) / 2).
  int tro[NDB];
  {
    const int r = 4 * lg + (li >> 2);
    const int fh = T::swz_v(r) / 2;
    const int base = r * ROWB + ((li >> 1) & 1) * 16 + (li & 1) * 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db) tro[db] = base + 32 * (db ^ fh);
  }

  auto compute = [&](int it, const unsigned char *kbuf, const unsigned char *vbuf) {
    const int t = it * NKQ + kq;
    const int j0 = t * BN;
    if (!(t < n_tiles && g_active && j0 <= g_kmax)) return;
    const unsigned char *kt = kbuf + kq * T::T_BYTES;
    const unsigned char *vt = vbuf + kq * T::T_BYTES;
    // ---- Sᵀ = K·Qᵀ - running max (log2 units), every K operand feeds NB
    // query blocks --------------------------------------------------------------
    f32x4_t s[NB][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kt + kb * 16 * ROWB + kro[ks]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s[nb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nb][ks], s[nb][kb], 0, 0, 0);
      }
    }
    const bool diag = j0 + BN - 1 > prefix + qg0;
    bf16x8_t pb[NB][BN / 32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // ---- causal mask (diagonal tiles only) -----------------------------------
      if (diag) [[unlikely]] {
        // key j0 + 16 kb + 4 lg + r is visible iff 16 kb + r <= lim
        const int lim = prefix + qg0 + nb * 16 + li - j0 - 4 * lg;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r > lim) s[nb][kb][r] = kNegInf;
      }
      // ---- lazy rescale: only a tile whose scores (scaled to log2 units)
      // exceed the running max by more than the slack moves it (the first
      // visible tile always does) --------------------------------------------
      float m0 = max3(s[nb][0][0], s[nb][0][1], s[nb][0][2]);
      m0 = max3(m0, s[nb][0][3], s[nb][1][0]);
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) {
        m0 = max3(m0, s[nb][kb][1], s[nb][kb][2]);
        m0 = kb + 1 < NKB ? max3(m0, s[nb][kb][3], s[nb][kb + 1][0])
                          : fmaxf(m0, s[nb][kb][3]);
      }
      // (scale > 0 commutes with the max; a masked score is -inf and never
      // passes the threshold, which is -inf before the first visible key)
      if (__any(m0 > thr[nb])) [[unlikely]] {
        const float mnew = fmaxf(mc[nb], quad_max(m0) * qk_scale);
        // a query with no visible key yet keeps max -inf: no rescale (and
        // no -inf - -inf)
        const float alpha = mnew == mc[nb] ? 1.f : fast_exp2(mc[nb] - mnew);
        mc[nb] = mnew;
        // every score of a query with max -inf is masked: any finite offset
        // gives p = 0 (and -mc would be +inf)
        nmc[nb] = mnew == kNegInf ? 0.f : -mnew;
        thr[nb] = (mnew + kRescaleSlack) / qk_scale;
        lacc[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[nb][db] *= alpha;
      }
#pragma unroll
      for (int t2 = 0; t2 < BN / 32; ++t2) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(fmaf(s[nb][2 * t2][r], qk_scale, nmc[nb]));
          p[4 + r] = fast_exp2(fmaf(s[nb][2 * t2 + 1][r], qk_scale, nmc[nb]));
        }
        const u32x4_t pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        pb[nb][t2] = as_bf16x8(pw);
      }
    }
    // ---- row sums and Oᵀ += Vᵀ·Pᵀ, every V operand feeds NB query blocks ---------
#pragma unroll
    for (int t2 = 0; t2 < BN / 32; ++t2) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        lacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[nb][t2], lacc[nb], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(vt + tro[db] + t2 * 32 * ROWB);
        const u32x2_t lo = read_tr16(src);
        const u32x2_t hi = read_tr16(src + 16 * ROWB / 2);
        const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8_t a = as_bf16x8(av);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nb][t2], o[nb][db], 0, 0, 0);
      }
    }
  };
  // the loads of an iteration are complete in every wave after this
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(0, kb0, vb0);
  sync();
  int it = 0;
  for (; it + 1 < n_iter; it += 2) {
    issue(it + 1, kb1, vb1);
    compute(it, kb0, vb0);
    sync();
    issue(it + 2, kb0, vb0);
    compute(it + 1, kb1, vb1);
    sync();
  }
  if (it < n_iter) {
    compute(it, kb0, vb0);
    sync();
  }

  // ---- merge the key quarters of each query group (log-sum-exp), store -----------
  // 1. running max and sum of every (group, query, quarter) -> mm, ml
  //    [NQG][NQW][NKQ] in vb0;
  // 2. each wave weights its own output by exp2(m - M) / L (M, L over the
  //    four quarters of the query) and writes it as fp32 [NKQ][NQW][D] into
  //    kb0 (group 0) / kb1 (group 1), 16-byte chunk c of row qi at position
  //    c ^ (qi % 16), so the 16 rows of one write fall on distinct banks;
  // 3. every thread adds the four quarters of 4 consecutive outputs and stores
  //    them as bf16.
  float *mm = mml;                    // [NQG][NQW][NKQ]
  float *ml = mm + NQG * NQW * NKQ;   // [NQG][NQW][NKQ]
  // fp32 output of (group, quarter): D = 64 puts a group's four quarters in
  // kb0 / kb1; D = 128 two per buffer, quarters 2 and 3 in vb0 / vb1
  constexpr int QBYTES = NQW * D * 4;
  constexpr int QPER = T::BUF / QBYTES;
  static_assert(QPER * QBYTES == T::BUF && NKQ % QPER == 0, "merge layout");
  auto quarter = [&](int grp, int kk) -> float * {
    unsigned char *bb = kk / QPER == 0 ? (grp == 0 ? kb0 : kb1) : (grp == 0 ? vb0 : vb1);
    return reinterpret_cast<float *>(bb + (kk % QPER) * QBYTES);
  };
  if (lg == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qi = nb * 16 + li;
      mm[(qgi * NQW + qi) * NKQ + kq] = mc[nb];
      ml[(qgi * NQW + qi) * NKQ + kq] = lacc[nb][0];
    }
  }
  __syncthreads();
  {
    float *mo = quarter(qgi, kq);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qi = nb * 16 + li;
      float m4[NKQ], l4[NKQ];
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk) {
        m4[kk] = mm[(qgi * NQW + qi) * NKQ + kk];
        l4[kk] = ml[(qgi * NQW + qi) * NKQ + kk];
      }
      float M = m4[0];
#pragma unroll
      for (int kk = 1; kk < NKQ; ++kk) M = fmaxf(M, m4[kk]);
      float L = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk)
        // a key part that saw no key of this query contributes nothing
        L = fmaf(m4[kk] == kNegInf ? 0.f : fast_exp2(m4[kk] - M), l4[kk], L);
      // (a query past the end of the sequence has L = 0; it is not stored)
      const float wgt = mc[nb] == kNegInf ? 0.f : fast_exp2(mc[nb] - M) / L;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4_t *>(mo + qi * D + (((db * 4 + lg) ^ li) * 4)) = o[nb][db] * wgt;
    }
  }
  __syncthreads();
  for (int i = tid; i < BM * D / 4; i += T::THREADS) {
    const int q = i / (D / 4);   // query inside the workgroup
    const int c = i % (D / 4);   // 16-byte chunk: outputs 4c .. 4c+3
    const int grp = q / NQW, qi = q % NQW;
    const int qglob = qt * BM + q;
    if (qglob >= Lq) continue;
    const int off = qi * D + ((c ^ (qi % 16)) * 4);
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(quarter(grp, 0) + off);
#pragma unroll
    for (int kk = 1; kk < NKQ; ++kk) acc += *reinterpret_cast<const f32x4_t *>(quarter(grp, kk) + off);
    *reinterpret_cast<u32x2_t *>(outg + ((size_t)j * Lq + qglob) * D + 4 * c) =
        u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

template <int D, bool PAGED, int BN = 4096 / D, int NKQ = 4>
hipError_t launch_lds(const PrefillArgs &a, hipStream_t stream) {
  using T = PT<D, BN, NKQ>;
  const int n_qtiles = (a.Lq + T::BM - 1) / T::BM;
  const int NH = a.B * a.Hq;
  const int heads_per_xcd = (NH + kXcds - 1) / kXcds;
  const long blocks = (long)kXcds * heads_per_xcd * n_qtiles;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  prefill_lds_kernel<D, PAGED, BN, NKQ><<<dim3((unsigned)blocks), T::THREADS, 0, stream>>>(
      static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
      static_cast<const uint16_t *>(a.v), static_cast<uint16_t *>(a.out), NH,
      a.Hq, a.Hkv, a.max_length, a.Lq, a.prefix_len, a.scale * kLog2e,
      n_qtiles, heads_per_xcd, a.block_table, a.max_blocks, a.page_size,
      a.num_pages, a.head_major);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  const bool paged = a.block_table != nullptr;
  // With at least two workgroups per CU to run, the half-LDS forms let two
  // of them share a CU out of step with each other (measured at D = 64: 32
  // heads of the prefill workload 43.6 us with 4 KiB tiles against 49.4 us);
  // with fewer, the full form halves the iterations (16 heads: 26.8 us
  // against 28.4 us).
  const long blocks = (long)kXcds * ((a.B * a.Hq + kXcds - 1) / kXcds) *
                      ((a.Lq + P64::BM - 1) / P64::BM);
  const bool two_per_cu = blocks >= 2L * kCUs;
  if (a.D == 128) {
    if (two_per_cu)
      return paged ? launch_lds<128, true, 32, 2>(a, stream) : launch_lds<128, false, 32, 2>(a, stream);
    return paged ? launch_lds<128, true>(a, stream) : launch_lds<128, false>(a, stream);
  }
  if (two_per_cu)
    return paged ? launch_lds<64, true, 32>(a, stream) : launch_lds<64, false, 32>(a, stream);
  return paged ? launch_lds<64, true>(a, stream) : launch_lds<64, false>(a, stream);
}

}  // namespace attn
