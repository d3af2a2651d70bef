// Top-k sparsified attention scores (gfx950).
//
// Operation: "c2psa multi-head self-attention high-concurrency inference",
// core implementation §2 — scores q·kᵀ with no scale, keep the topk largest
// of every row, zero the others, multiply the sparse matrix by v; no softmax.
// Equal scores at the boundary go to the lower key index.
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
//      a) the k-th largest fp32-rounded score T by a most-significant-digit
//         radix select over the 32-bit order-preserving key: four passes of
//         8 bits, each a 256-bin LDS histogram of the keys still sharing the
//         prefix, a wave prefix sum over the bins from the top and a ballot
//         for the bin holding the k-th key. Every score whose fp32 key
//         exceeds T is in (rounding is monotone);
//      b) only if more scores share T than places remain, a bisection over
//         the exact 64-bit keys of those candidates, and remaining ties are
//         filled in ascending key index.
//      The chosen (index, score) pairs are compacted in ascending index order
//      (into the row's own LDS storage and a per-wave index list).
//   3. gather: lanes = 4 slot groups x 16 groups of 4 dimensions; each slot
//      group walks every 4th selected key and adds score * v[key] in fp64
//      (one coalesced 256-byte row read per key per slot group, 16 in flight);
//      the four partial sums are added across lanes and rounded to fp32.
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

// Inclusive prefix sum over the 64 lanes: DPP row shifts inside each
// 16-lane row (out-of-row sources contribute 0), then the totals of the
// earlier rows read with readlane.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, int lane) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t t1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? t0 : 0u) + (lane >= 32 ? t1 : 0u) + (lane >= 48 ? t2 : 0u);
}

// LDS writes of the wave become visible to all its lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t order64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int NTP>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const float *__restrict__ qg, const float *__restrict__ kg,
    const float *__restrict__ vg, float *__restrict__ outg,
    int32_t *__restrict__ idxg, int n, int topk, int n_qtiles, int n_work) {
  constexpr int NP = 64 * NTP;  // padded row length
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double *S = reinterpret_cast<double *>(smem);                 // [QB][NP]
  int *jl = reinterpret_cast<int *>(smem + (size_t)QB * NP * 8);  // [4][NP]
  __shared__ __attribute__((aligned(16))) uint32_t hst[4 * 256];  // per-wave histograms
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
    const int nkb = (n + 15) / 16;
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
    if (row_ok) {
      // ---- 2. select ---------------------------------------------------------------
      double s[NTP];
      uint32_t k32[NTP];
#pragma unroll
      for (int t = 0; t < NTP; ++t) {
        // computed for every slot (padding too: in bounds, maybe stale) and
        // then selected, so that no load waits behind a branch
        const double v = S[i * NP + l + 64 * t] + 0.0;  // +0.0 turns -0 into +0
        const uint32_t key = order32((float)v + 0.0f);
        const bool ok = l + 64 * t < n;
        s[t] = ok ? v : 0.0;
        k32[t] = ok ? key : 0u;
      }
      // k-th largest 32-bit key by 4 radix passes of 8 bits, most
      // significant first: histogram the candidates' digit in LDS, scan
      // the bins from the top, keep the bin that holds the k-th key.
      uint32_t T = 0;        // key prefix found so far
      int krem = topk;       // rank still to find inside the prefix
      int gt = 0;            // keys above the prefix
      int nc = 0;            // keys equal to the final key
      uint32_t *hist = hst + w * 256;
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
          const bool cand = k32[t] != 0u &&
                            (pass == 0 || (k32[t] >> (shift + 8)) == T);
          if (cand) atomicAdd(&hist[(k32[t] >> shift) & 0xffu], 1u);
        }
        wave_sync();
        // lane l holds bins 255-4l (top) .. 252-4l
        const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(&hist[252 - 4 * l]);
        const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
        const uint32_t incl = wave_inclusive_scan(local, l);
        const uint64_t hit = __ballot(incl >= (uint32_t)krem);
        const int L = __ffsll((unsigned long long)hit) - 1;
        uint32_t c = __builtin_amdgcn_readlane(incl - local, L);
        const uint32_t h3 = __builtin_amdgcn_readlane(hv[3], L);
        const uint32_t h2 = __builtin_amdgcn_readlane(hv[2], L);
        const uint32_t h1 = __builtin_amdgcn_readlane(hv[1], L);
        const uint32_t h0 = __builtin_amdgcn_readlane(hv[0], L);
        int bin, hb;
        if (c + h3 >= (uint32_t)krem) { bin = 255 - 4 * L; hb = h3; }
        else if ((c += h3) + h2 >= (uint32_t)krem) { bin = 254 - 4 * L; hb = h2; }
        else if ((c += h2) + h1 >= (uint32_t)krem) { bin = 253 - 4 * L; hb = h1; }
        else { c += h1; bin = 252 - 4 * L; hb = h0; }
        krem -= (int)c;
        gt += (int)c;
        T = (T << 8) | (uint32_t)bin;
        nc = hb;
        *reinterpret_cast<u32x4_t *>(&hist[252 - 4 * l]) = u32x4_t{0u, 0u, 0u, 0u};
        wave_sync();
      }
      uint64_t selm[NTP], cm[NTP];
#pragma unroll
      for (int t = 0; t < NTP; ++t) {
        selm[t] = __ballot(k32[t] > T);
        cm[t] = __ballot(k32[t] == T);
      }
      const int need = topk - gt;  // >= 1
      if (nc == need) {
#pragma unroll
        for (int t = 0; t < NTP; ++t) selm[t] |= cm[t];
      } else {
        // Exact fp64 order among the candidates sharing the fp32 key T.
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
      // before accumulating (one memory latency per chunk); slots past topk
      // read row 0 and contribute nothing.
      auto chunk = [&](int p0, auto full) {
        constexpr bool FULL = decltype(full)::value;  // all 64 slots < topk
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
          const int j = (FULL || p0 + sg + 4 * u < topk) ? jr[u] : 0;
          vv[u] = *reinterpret_cast<const float4 *>(vb + (size_t)j * DIM + 4 * dq);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          // a slot past topk adds fma(0, 0, acc) = acc exactly
          const bool ok = FULL || p0 + sg + 4 * u < topk;
          const double sv = ok ? sj[u] : 0.0;
          const float4 x = ok ? vv[u] : float4{0.f, 0.f, 0.f, 0.f};
          acc[0] = fma(sv, (double)x.x, acc[0]);
          acc[1] = fma(sv, (double)x.y, acc[1]);
          acc[2] = fma(sv, (double)x.z, acc[2]);
          acc[3] = fma(sv, (double)x.w, acc[3]);
        }
      };
      int p0 = 0;
      for (; p0 + 64 <= topk; p0 += 64) chunk(p0, std::true_type{});
      if (p0 < topk) chunk(p0, std::false_type{});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
      }
      if (sg == 0) {
        const float4 o = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
        *reinterpret_cast<float4 *>(outg + (bh * n + qr) * DIM + 4 * dq) = o;
      }
    }
    wave_sync();
  }
}

template <int NTP>
hipError_t launch_ntp(const TopkArgs &a, hipStream_t stream) {
  const size_t shmem = (size_t)64 * NTP * (QB * 8 + 4 * 4);
  if (shmem > 65536) {  // opt in to more than 64 KiB of LDS (gfx950: 160 KiB)
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&topk_kernel<NTP>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const int n_qtiles = (a.n + QB - 1) / QB;
  const int n_work = n_qtiles * a.h * a.b;  // <= 2^23, checked by the caller
  topk_kernel<NTP><<<n_work, kThreads, shmem, stream>>>(
      a.q, a.k, a.v, a.out, a.idx, a.n, a.topk, n_qtiles, n_work);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
  const int nt = (a.n + 63) / 64;
  if (nt <= 1) return launch_ntp<1>(a, stream);
  if (nt <= 2) return launch_ntp<2>(a, stream);
  if (nt <= 4) return launch_ntp<4>(a, stream);
  if (nt <= 8) return launch_ntp<8>(a, stream);
  return launch_ntp<16>(a, stream);
}

}  // namespace attn
