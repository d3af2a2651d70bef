// Top-k sparsified attention scores (gfx950).
//
// Operation: "c2psa multi-head self-attention high-concurrency inference",
// core implementation §2 — scores q·kᵀ with no scale, keep the topk largest
// of every row, zero the others, multiply the sparse matrix by v; no softmax.
// Equal scores at the boundary go to the lower key index.
//
// Decoder form (same page, further thoughts): row i chooses only among keys
// j <= i. A row with i+1 <= topk keeps all of them; a longer row keeps its
// topk/2 most recent keys and chooses the other topk - topk/2 by score among
// the older ones j <= i - topk/2. The score blocks past a workgroup's last
// row are not computed.
//
// Precision: every fp32·fp32 product is exact in fp64, so scores and the
// output sum are accumulated in fp64 and the selection is made on the fp64
// scores; the output is rounded once to fp32.
//
// One workgroup = 4 waves = 16 query rows of one (b, h):
//   1. scores: S[16][n] with v_mfma_f64_16x16x4_f64 (A = the 16 query rows,
//      B = 16 key rows per block; the 64 dimensions are spread as 16 MFMAs of
//      4), written to LDS. Waves take key blocks round-robin.
//   2. select, one row per wave at a time, lane e holding keys e, e+64, ...:
//      a) the row's score range (fp32-rounded, wave-wide max/min over DPP
//         and permlane swaps) defines a monotone map of the scores onto 256
//         buckets; a 256-bin LDS histogram scanned from the top gives the
//         bucket B holding the topk-th largest score: every score in a higher
//         bucket is taken;
//      b) the candidates in B are ranked exactly (fp64 score descending, key
//         index ascending) against each other with lane reads, and the first
//         topk - (scores above B) are taken; if more than 64 scores share B
//         (equal or nearly equal scores), a bisection over their exact 64-bit
//         order keys decides instead, remaining ties in ascending key index.
//      The chosen (index, score) pairs are compacted in ascending index order
//      (into the row's own LDS storage and a per-wave index list).
//   3. gather: lanes = 4 slot groups x 16 groups of 4 dimensions; each slot
//      group walks every 4th selected key and adds score * v[key] in fp64
//      (one coalesced 256-byte row read per key per slot group, 16 in flight);
//      the four partial sums are added across the lane rows in registers
//      (permlane swaps) and rounded to fp32.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int QB = 16;  // query rows per workgroup
constexpr int DIM = 64;

__device__ __forceinline__ uint32_t order32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// LDS writes of the wave become visible to all its lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum / minimum over the 64 lanes without LDS round trips: DPP moves
// inside each 16-lane row (swap neighbours, swap pairs, mirror the 8-lane
// halves, mirror the row), then v_permlane16_swap / v_permlane32_swap across
// rows.
template <bool MAX>
__device__ __forceinline__ float wave_extreme(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
#define ATTN_DPP(v, ctrl) \
  __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false))
  x = op(x, ATTN_DPP(x, 0xB1));   // quad_perm [1,0,3,2]
  x = op(x, ATTN_DPP(x, 0x4E));   // quad_perm [2,3,0,1]
  x = op(x, ATTN_DPP(x, 0x141));  // row_half_mirror
  x = op(x, ATTN_DPP(x, 0x140));  // row_mirror
#undef ATTN_DPP
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// x of this lane plus x of lane l ^ 16 (ROW2 false) or l ^ 32 (true): the
// 16-lane rows of the wave swapped in registers (v_permlane16_swap /
// v_permlane32_swap on both 32-bit halves), no LDS round trip. The swap
// hands each lane the pair {x_l, x_partner} in either order; the sum is the
// same either way.
template <bool ROW2>
__device__ __forceinline__ double add_row_partner(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto a = ROW2 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                      : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto c = ROW2 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                      : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const double d0 = __longlong_as_double((long long)(((uint64_t)c[0] << 32) | a[0]));
  const double d1 = __longlong_as_double((long long)(((uint64_t)c[1] << 32) | a[1]));
  return d0 + d1;
}

__device__ __forceinline__ uint64_t order64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int NTP, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const float *__restrict__ qg, const float *__restrict__ kg,
    const float *__restrict__ vg, float *__restrict__ outg,
    int32_t *__restrict__ idxg, int n, int topk, int n_qtiles, int n_work) {
  constexpr int NP = 64 * NTP;  // padded row length
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double *S = reinterpret_cast<double *>(smem);                 // [QB][NP]
  int *jl = reinterpret_cast<int *>(smem + (size_t)QB * NP * 8);  // [4][NP]
  __shared__ __attribute__((aligned(16))) uint32_t hst[4 * 256];  // per-wave histograms
  __shared__ double cand_s[4 * 64];  // per-wave boundary candidates (score,
  __shared__ int cand_j[4 * 64];     // key index)
  for (int i = threadIdx.x; i < 4 * 256; i += kThreads) hst[i] = 0u;

  // Workgroup i runs on XCD i % 8. Each XCD takes a contiguous range of the
  // (b·h, query tile) work list, so the query tiles of one (b, h) share that
  // XCD's L2 and its K and V are fetched from HBM about once.
  const int xcd = blockIdx.x % 8;
  const int per = n_work / 8, extra = n_work % 8;
  const int work = xcd * per + min(xcd, extra) + (int)(blockIdx.x / 8);
  const size_t bh = (size_t)(work / n_qtiles);
  const int q0 = (work % n_qtiles) * QB;
  const float *qb = qg + bh * n * DIM;
  const float *kb = kg + bh * n * DIM;
  const float *vb = vg + bh * n * DIM;
  const int tid = threadIdx.x;
  const int w = tid / 64;
  const int l = tid % 64;
  const int li = l % 16;
  const int lg = l / 16;

  // ---- 1. scores ---------------------------------------------------------------
  // Query rows and key rows past n are read from row n-1 (in bounds); the
  // scores they produce sit in rows and columns that are never used.
  {
    double qa[16];
    {
      const int qr = min(q0 + li, n - 1);
      float4 x[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        x[c] = *reinterpret_cast<const float4 *>(qb + (size_t)qr * DIM + 16 * lg + 4 * c);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qa[4 * c + 0] = x[c].x;
        qa[4 * c + 1] = x[c].y;
        qa[4 * c + 2] = x[c].z;
        qa[4 * c + 3] = x[c].w;
      }
    }
    // causal: the block's rows see no key past its last row
    const int nkb = ((CAUSAL ? min(n, q0 + QB) : n) + 15) / 16;
    // Two accumulators halve the dependent MFMA chain (the 64-term sum is
    // split into two halves of 32).
    auto load_kblk = [&](int blk, float4 (&x)[4]) {
      const int kr = min(blk * 16 + li, n - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        x[c] = *reinterpret_cast<const float4 *>(kb + (size_t)kr * DIM + 16 * lg + 4 * c);
    };
    auto compute = [&](int blk, const float4 (&x4)[4]) {
      f64x4_t a0 = {0.0, 0.0, 0.0, 0.0}, a1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float4 x = x4[c], y = x4[c + 2];
        a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 0], (double)x.x, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 8], (double)y.x, a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 1], (double)x.y, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 9], (double)y.y, a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 2], (double)x.z, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 10], (double)y.z, a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 3], (double)x.w, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[4 * c + 11], (double)y.w, a1, 0, 0, 0);
      }
      // lane l, register r holds query row lg + 4r, key blk*16 + li
      if (blk < nkb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(lg + 4 * r) * NP + blk * 16 + li] = a0[r] + a1[r];
      }
    };
    // Two register buffers: each block's rows are loaded one block ahead of
    // their use. Blocks past the end are computed from clamped rows and not
    // stored. The scheduling barriers keep the compiler from sinking the
    // loads down to their use.
    float4 xa[4], xb[4];
    load_kblk(w, xa);
    for (int blk = w; blk < nkb; blk += 8) {
      load_kblk(blk + 4, xb);
      __builtin_amdgcn_sched_barrier(0);
      compute(blk, xa);
      load_kblk(blk + 8, xa);
      __builtin_amdgcn_sched_barrier(0);
      compute(blk + 4, xb);
    }
  }
  __syncthreads();

  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));  // lanes < l

  for (int ii = 0; ii < 4; ++ii) {
    const int i = 4 * w + ii;  // row inside the block
    const int qr = q0 + i;
    const bool row_ok = qr < n;  // uniform over the wave
    // Keys the row keeps. Causal: a row with qr + 1 <= topk keeps every
    // j <= qr; a longer one keeps its topk/2 most recent keys and chooses
    // the other topk - topk/2 by score among the older keys j < lim.
    const int cnt = CAUSAL ? min(topk, qr + 1) : topk;
    const bool dense = CAUSAL && qr + 1 <= topk;
    const int lim = CAUSAL ? qr + 1 - topk / 2 : n;
    const int kk = CAUSAL ? topk - topk / 2 : topk;  // chosen by score
    if (row_ok) {
      // ---- 2. select ---------------------------------------------------------------
      double s[NTP];
#pragma unroll
      for (int t = 0; t < NTP; ++t)  // every slot (padding too: in bounds, maybe stale)
        s[t] = S[i * NP + l + 64 * t] + 0.0;  // +0.0 turns -0 into +0
      uint64_t selm[NTP];
      if (dense) {
#pragma unroll
        for (int t = 0; t < NTP; ++t) selm[t] = __ballot(l + 64 * t <= qr);
      } else {
        bool ok[NTP];
        float mxf = -__builtin_inff(), mnf = __builtin_inff();
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
          ok[t] = l + 64 * t < lim;
          mxf = fmaxf(mxf, ok[t] ? (float)s[t] : -__builtin_inff());
          mnf = fminf(mnf, ok[t] ? (float)s[t] : __builtin_inff());
        }
        // (fp32-rounded range: any constants give a monotone map below)
        const double mx = wave_extreme<true>(mxf), mn = wave_extreme<false>(mnf);
        // Bucket of a score: a non-decreasing map of about [mn, mx] onto
        // 0..255 (correctly rounded fma, truncation and clamping are all
        // monotone), so a higher bucket means a strictly larger score. Equal
        // scores share a bucket; a row of (nearly) equal scores is all bucket 0.
        const double span = mx - mn;
        const double bs = span > 1e-290 ? 256.0 / span : 0.0;
        const double b0 = -mn * bs;
        int bk[NTP];
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
          const int bb = (int)fma(s[t], bs, b0);
          bk[t] = ok[t] ? min(max(bb, 0), 255) : -1;
        }
        // 256-bin histogram, scanned from the top: bucket B holds the topk-th
        // largest score, gt scores lie in higher buckets, nc in B.
        uint32_t *hist = hst + w * 256;
#pragma unroll
        for (int t = 0; t < NTP; ++t)
          if (bk[t] >= 0) atomicAdd(&hist[bk[t]], 1u);
        wave_sync();
        int B, gt, nc;
        {
          // lane l holds bins 255-4l (top) .. 252-4l
          const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(&hist[252 - 4 * l]);
          const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
          const uint32_t incl = wave_inclusive_scan(local, l);
          const uint64_t hit = __ballot(incl >= (uint32_t)kk);
          const int L = __ffsll((unsigned long long)hit) - 1;
          uint32_t c = __builtin_amdgcn_readlane(incl - local, L);
          const uint32_t h3 = __builtin_amdgcn_readlane(hv[3], L);
          const uint32_t h2 = __builtin_amdgcn_readlane(hv[2], L);
          const uint32_t h1 = __builtin_amdgcn_readlane(hv[1], L);
          const uint32_t h0 = __builtin_amdgcn_readlane(hv[0], L);
          int hb;
          if (c + h3 >= (uint32_t)kk) { B = 255 - 4 * L; hb = h3; }
          else if ((c += h3) + h2 >= (uint32_t)kk) { B = 254 - 4 * L; hb = h2; }
          else if ((c += h2) + h1 >= (uint32_t)kk) { B = 253 - 4 * L; hb = h1; }
          else { c += h1; B = 252 - 4 * L; hb = h0; }
          gt = (int)c;
          nc = hb;
          *reinterpret_cast<u32x4_t *>(&hist[252 - 4 * l]) = u32x4_t{0u, 0u, 0u, 0u};
        }
        uint64_t cm[NTP];
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
          selm[t] = __ballot(bk[t] > B);
          cm[t] = __ballot(bk[t] == B);
        }
        const int need = kk - gt;  // 1 <= need <= nc
        if (nc == need) {
#pragma unroll
          for (int t = 0; t < NTP; ++t) selm[t] |= cm[t];
        } else if (nc <= 64) {
          // The boundary bucket's candidates go to a per-wave list; each is
          // ranked by (score descending, index ascending) and the candidate of
          // rank need-1 is the last one taken.
          double *cs = cand_s + w * 64;
          int *cj = cand_j + w * 64;
          int before = 0;
#pragma unroll
          for (int t = 0; t < NTP; ++t) {
            if ((cm[t] >> l) & 1ull) {
              const int pos = before + __popcll(cm[t] & below);
              cs[pos] = s[t];
              cj[pos] = l + 64 * t;
            }
            before += __popcll(cm[t]);
          }
          wave_sync();
          const double my_s = cs[l < nc ? l : 0];
          const int my_j = cj[l < nc ? l : 0];
          // candidate m is in lane m: broadcast it with lane reads
          const int my_lo = (int)(uint32_t)__double_as_longlong(my_s);
          const int my_hi = (int)(uint32_t)(__double_as_longlong(my_s) >> 32);
          int rank = 0;
          for (int m = 0; m < nc; ++m) {
            const uint64_t ob = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_hi, m) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane(my_lo, m);
            const double os = __longlong_as_double((long long)ob);
            const int oj = __builtin_amdgcn_readlane(my_j, m);
            rank += (os > my_s || (os == my_s && oj < my_j)) ? 1 : 0;
          }
          const uint64_t last = __ballot(l < nc && rank == need - 1);
          const int Ll = __ffsll((unsigned long long)last) - 1;
          // (Ll is the same in every lane: lane reads, no LDS round trip)
          const double ts = __longlong_as_double(
              (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_hi, Ll) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane(my_lo, Ll)));
          const int tj = __builtin_amdgcn_readlane(my_j, Ll);
#pragma unroll
          for (int t = 0; t < NTP; ++t)
            selm[t] |= __ballot(((cm[t] >> l) & 1ull) &&
                                (s[t] > ts || (s[t] == ts && l + 64 * t <= tj)));
          wave_sync();
        } else {
          // Many equal or nearly equal scores: exact fp64 order among the
          // candidates by a bisection over their 64-bit order keys.
          uint64_t k64[NTP];
#pragma unroll
          for (int t = 0; t < NTP; ++t)
            k64[t] = ((cm[t] >> l) & 1ull) ? order64(s[t]) : 0ull;
          uint64_t T2 = 0;
          for (int bit = 63; bit >= 0; --bit) {
            const uint64_t cand = T2 | (1ull << bit);
            int cnt = 0;
#pragma unroll
            for (int t = 0; t < NTP; ++t) cnt += __popcll(__ballot(k64[t] >= cand));
            if (cnt >= need) T2 = cand;
          }
          int need2 = need;
#pragma unroll
          for (int t = 0; t < NTP; ++t) {
            const uint64_t m = __ballot(k64[t] > T2);
            selm[t] |= m;
            need2 -= __popcll(m);
          }
          // ties at T2: ascending key index = slot-major, lane-minor
          for (int t = 0; t < NTP; ++t) {
            uint64_t tm = __ballot(k64[t] == T2);
            while (need2 > 0 && tm) {
              const uint64_t low = tm & (~tm + 1ull);
              selm[t] |= low;
              tm ^= low;
              --need2;
            }
          }
        }
        if (CAUSAL) {  // the most recent keys lim..qr
#pragma unroll
          for (int t = 0; t < NTP; ++t)
            selm[t] |= __ballot(l + 64 * t >= lim && l + 64 * t <= qr);
        }
      }  // !dense
      // compact the chosen (index, score) pairs in ascending index order
      int before = 0;
#pragma unroll
      for (int t = 0; t < NTP; ++t) {
        const uint64_t mt = selm[t];
        if ((mt >> l) & 1ull) {
          const int pos = before + __popcll(mt & below);
          const int j = l + 64 * t;
          jl[w * NP + pos] = j;
          S[i * NP + pos] = s[t];
          if (idxg) idxg[(bh * n + qr) * (size_t)topk + pos] = j;
        }
        before += __popcll(mt);
      }
      if (CAUSAL && idxg)  // rows keeping fewer than topk keys: pad with -1
        for (int p = cnt + l; p < topk; p += 64) idxg[(bh * n + qr) * (size_t)topk + p] = -1;
    }
    // From here on every LDS word a wave touches is its own (row i of S and
    // its index list), so the lanes of the wave only need to see each other.
    wave_sync();
    if (row_ok) {
      // ---- 3. gather ---------------------------------------------------------------
      const int sg = l / 16;
      const int dq = l % 16;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      // chunks of 64 selected keys: each slot group issues its 16 row loads
      // before accumulating (one memory latency per chunk); slots past the
      // row's key count read row 0 and contribute nothing.
      auto chunk = [&](int p0, auto full) {
        constexpr bool FULL = decltype(full)::value;  // all 64 slots < cnt
        float4 vv[16];
        double sj[16];
        int jr[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {  // p < NP: in bounds, maybe stale
          jr[u] = jl[w * NP + p0 + sg + 4 * u];
          sj[u] = S[i * NP + p0 + sg + 4 * u];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int j = (FULL || p0 + sg + 4 * u < cnt) ? jr[u] : 0;
          vv[u] = *reinterpret_cast<const float4 *>(vb + (size_t)j * DIM + 4 * dq);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          // a slot past cnt adds fma(0, 0, acc) = acc exactly
          const bool ok = FULL || p0 + sg + 4 * u < cnt;
          const double sv = ok ? sj[u] : 0.0;
          const float4 x = ok ? vv[u] : float4{0.f, 0.f, 0.f, 0.f};
          acc[0] = fma(sv, (double)x.x, acc[0]);
          acc[1] = fma(sv, (double)x.y, acc[1]);
          acc[2] = fma(sv, (double)x.z, acc[2]);
          acc[3] = fma(sv, (double)x.w, acc[3]);
        }
      };
      int p0 = 0;
      for (; p0 + 64 <= cnt; p0 += 64) chunk(p0, std::true_type{});
      if (p0 < cnt) chunk(p0, std::false_type{});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = add_row_partner<false>(acc[e]);
        acc[e] = add_row_partner<true>(acc[e]);
      }
      if (sg == 0) {
        const float4 o = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
        *reinterpret_cast<float4 *>(outg + (bh * n + qr) * DIM + 4 * dq) = o;
      }
    }
    wave_sync();
  }
}

template <int NTP, bool CAUSAL>
hipError_t launch_ntp(const TopkArgs &a, hipStream_t stream) {
  const size_t shmem = (size_t)64 * NTP * (QB * 8 + 4 * 4);
  if (shmem > 65536) {  // opt in to more than 64 KiB of LDS (gfx950: 160 KiB)
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&topk_kernel<NTP, CAUSAL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const int n_qtiles = (a.n + QB - 1) / QB;
  const int n_work = n_qtiles * a.h * a.b;  // <= 2^23, checked by the caller
  topk_kernel<NTP, CAUSAL><<<n_work, kThreads, shmem, stream>>>(
      a.q, a.k, a.v, a.out, a.idx, a.n, a.topk, n_qtiles, n_work);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_causal(const TopkArgs &a, hipStream_t stream) {
  const int nt = (a.n + 63) / 64;
  if (nt <= 1) return launch_ntp<1, CAUSAL>(a, stream);
  if (nt <= 2) return launch_ntp<2, CAUSAL>(a, stream);
  if (nt <= 4) return launch_ntp<4, CAUSAL>(a, stream);
  if (nt <= 8) return launch_ntp<8, CAUSAL>(a, stream);
  return launch_ntp<16, CAUSAL>(a, stream);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
  return a.causal ? launch_causal<true>(a, stream) : launch_causal<false>(a, stream);
}

}  // namespace attn
