// Causal prefill against a cached prefix on bf16 matrix cores (gfx950).
//
// Operation: "step14_3 — batched attention: removing the per-head Python
// loop", solution section — for every head at once, scores = Q·Kᵀ scaled by
// 1/sqrt(d_head), causal entries set to -inf, softmax over each row, times V;
// the going-further section fuses the three steps into one kernel so the
// score matrix never reaches HBM. New token i sits at cache row prefix+i and
// sees rows [0, prefix+i].
//
// One workgroup = 4 waves = 64 queries (16 per wave) of one head, walking
// 64-key tiles up to the causal bound of its last query.
//   * Block -> work map: workgroup id i runs on XCD i % 8. Every query tile
//     of one head goes to the same XCD, so the head's K and V are fetched
//     from HBM once into that XCD's L2 and re-read from there by its 16
//     query tiles; on each XCD the tiles run longest (most keys) first.
//   * K is read straight from L1/L2 into the A-operand registers of
//     v_mfma_f32_16x16x32_bf16 (16 key rows x 32 dims per instruction); V is
//     staged once per tile in LDS, transposed (d-major), shared by the 4 waves
//     and double-buffered. The next tile's K and V loads are issued before the
//     current tile is computed.
//   * Sᵀ = K·Qᵀ puts each lane on one query and 4 keys of every 16-key block:
//     the exact operand layout of Oᵀ += Vᵀ·Pᵀ, so P never leaves registers.
//   * Softmax in the exp2 domain: the running max is kept on the raw scores
//     (scale > 0 commutes with max), p = exp2(fma(s, scale*log2 e, -m)); the
//     output is rescaled only when the running max grows by more than 8 (in
//     log2 units), so p stays below 2^8 and most tiles skip the rescale. Row
//     sums come from the matrix cores too: an all-ones A operand times Pᵀ
//     gives every query's sum of the same bf16 probabilities the output uses.
//   * Only tiles that cross the diagonal evaluate the mask; tiles past a
//     wave's last visible key are skipped.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 64;  // queries per workgroup
constexpr int BN = 64;  // keys per tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int D>
struct Tile {
  static constexpr int KS = D / 32;    // MFMA k-steps of K·Qᵀ
  static constexpr int NDB = D / 16;   // 16-wide output blocks
  static constexpr int NKB = BN / 16;  // 16-key blocks per tile
  static constexpr int SV = BN + 4;    // Vᵀ row stride in LDS (elements)
  static constexpr int VCH = (BN / 2) * (D / 8) / kThreads;  // V items per thread
  static_assert(VCH >= 1, "tile too small for the workgroup");
};

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t *__restrict__ qg, const uint16_t *__restrict__ kg,
    const uint16_t *__restrict__ vg, uint16_t *__restrict__ outg, int NH,
    int Hq, int Hkv, int max_length, int Lq, int prefix, float qk_scale,
    int n_qtiles, int heads_per_xcd) {
  using T = Tile<D>;
  constexpr int KS = T::KS, NDB = T::NDB, NKB = T::NKB, SV = T::SV;
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * SV];

  // ---- work item: (head instance, query tile) -----------------------------------
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int k = id / kXcds;
  const int j = xcd + kXcds * (k % heads_per_xcd);  // head instance b*Hq + h
  if (j >= NH) return;
  const int qt = n_qtiles - 1 - k / heads_per_xcd;  // longest tiles first
  const int b = j / Hq;
  const int h = j % Hq;
  const int kvh = h / (Hq / Hkv);

  const int tid = threadIdx.x;
  const int w = tid / 64;
  const int l = tid % 64;
  const int li = l % 16;
  const int lg = l / 16;

  const int kv_len = prefix + Lq;
  const int q_end = min((qt + 1) * BM, Lq);
  const int n_tiles = (prefix + q_end + BN - 1) / BN;
  const int qw0 = qt * BM + w * 16;     // first query of this wave
  const int qme = qw0 + li;             // this lane's query
  const bool w_active = qw0 < Lq;
  const int w_kmax = prefix + min(qw0 + 15, Lq - 1);  // last key the wave sees
  const int jlim = prefix + qme;        // last key this lane's query sees

  const size_t kvbase = ((size_t)b * Hkv + kvh) * (size_t)max_length * D;
  const uint16_t *kbase = kg + kvbase;
  const uint16_t *vbase = vg + kvbase;

  bf16x8_t qf[KS];
  {
    const size_t qrow = ((size_t)j * Lq + (size_t)qme) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qme < Lq) v = *reinterpret_cast<const u32x4_t *>(qg + qrow + ks * 32 + 8 * lg);
      qf[ks] = as_bf16x8(v);
    }
  }
  const u32x4_t ones_w = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8_t ones = as_bf16x8(ones_w);

  f32x4_t o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};  // row sums (4 identical copies)
  float mc = kNegInf;                   // running max, scaled (log2 units)

  u32x4_t kf[NKB][KS];
  u32x4_t vreg[T::VCH][2];

  auto load_k = [&](int t, u32x4_t (&dst)[NKB][KS]) {
    const int j0 = t * BN;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = j0 + kb * 16 + li;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row < kv_len)
          v = *reinterpret_cast<const u32x4_t *>(kbase + (size_t)row * D + ks * 32 + 8 * lg);
        dst[kb][ks] = v;
      }
    }
  };
  auto load_v = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) {
      const int c = tid + i * kThreads;
      const int col = (c % (D / 8)) * 8;
      const int r0 = j0 + 2 * (c / (D / 8));
      u32x4_t a = {0u, 0u, 0u, 0u}, bb = {0u, 0u, 0u, 0u};
      if (r0 < kv_len)
        a = *reinterpret_cast<const u32x4_t *>(vbase + (size_t)r0 * D + col);
      if (r0 + 1 < kv_len)
        bb = *reinterpret_cast<const u32x4_t *>(vbase + (size_t)(r0 + 1) * D + col);
      vreg[i][0] = a;
      vreg[i][1] = bb;
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) {
      const int c = tid + i * kThreads;
      const int col = (c % (D / 8)) * 8;
      const int p = c / (D / 8);  // row pair inside the tile
      const u32x4_t a = vreg[i][0], bb = vreg[i][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (a[e] & 0xffffu) | (bb[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (bb[e] & 0xffff0000u);
        *reinterpret_cast<uint32_t *>(&Vt[buf][(col + 2 * e) * SV + 2 * p]) = lo;
        *reinterpret_cast<uint32_t *>(&Vt[buf][(col + 2 * e + 1) * SV + 2 * p]) = hi;
      }
    }
  };

  load_v(0);
  load_k(0, kf);
  store_v(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < n_tiles;
    u32x4_t kn[NKB][KS];
    if (more) {
      load_v(t + 1);
      load_k(t + 1, kn);
    }
    const int j0 = t * BN;
    if (w_active && j0 <= w_kmax) {
      // ---- Sᵀ = K·Qᵀ (raw scores) ----------------------------------------------------
      f32x4_t s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kb][ks]),
                                                         qf[ks], s[kb], 0, 0, 0);
      }
      // ---- causal mask (diagonal tiles only) and row max ---------------------
      if (j0 + BN - 1 > prefix + qw0) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j0 + kb * 16 + 4 * lg + r > jlim) s[kb][r] = kNegInf;
      }
      float mloc = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        mloc = fmaxf(fmaxf(mloc, fmaxf(s[kb][0], s[kb][1])), fmaxf(s[kb][2], s[kb][3]));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mloc_c = mloc * qk_scale;
      if (__any(mloc_c > mc + kRescaleSlack)) {
        const float mnew = fmaxf(mc, mloc_c);
        const float alpha = fast_exp2(mc - mnew);
        mc = mnew;
        lacc *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      }
      // ---- P, row sums and Oᵀ += Vᵀ·Pᵀ ----------------------------------------
      const float nmc = -mc;
#pragma unroll
      for (int t2 = 0; t2 < BN / 32; ++t2) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(fmaf(s[2 * t2][r], qk_scale, nmc));
          p[4 + r] = fast_exp2(fmaf(s[2 * t2 + 1][r], qk_scale, nmc));
        }
        const u32x4_t pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        const bf16x8_t pb = as_bf16x8(pw);
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, lacc, 0, 0, 0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t *vrow = &Vt[buf][(db * 16 + li) * SV + 32 * t2 + 4 * lg];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + 16);
          const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), pb,
                                                         o[db], 0, 0, 0);
        }
      }
    }
    if (more) {
      store_v(buf ^ 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = kn[kb][ks];
    }
    __syncthreads();
  }

  // ---- finalise: divide by the row sum, store bf16 -------------------------------
  if (qme < Lq) {
    const float inv = 1.f / lacc[0];
    uint16_t *orow = outg + ((size_t)j * Lq + (size_t)qme) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2_t wv = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                          pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
      *reinterpret_cast<u32x2_t *>(orow + db * 16 + 4 * lg) = wv;
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream) {
  const int n_qtiles = (a.Lq + BM - 1) / BM;
  const int NH = a.B * a.Hq;
  const int heads_per_xcd = (NH + kXcds - 1) / kXcds;
  const long blocks = (long)kXcds * heads_per_xcd * n_qtiles;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  prefill_kernel<D><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(
      static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
      static_cast<const uint16_t *>(a.v), static_cast<uint16_t *>(a.out), NH,
      a.Hq, a.Hkv, a.max_length, a.Lq, a.prefix_len, a.scale * kLog2e,
      n_qtiles, heads_per_xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace attn
