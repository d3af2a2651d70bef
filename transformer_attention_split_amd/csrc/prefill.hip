// Causal prefill against a cached prefix on bf16 matrix cores (gfx950).
//
// Operation: "step14_3 — batched attention: removing the per-head Python
// loop", solution section — for every head at once, scores = Q·Kᵀ scaled by
// 1/sqrt(d_head), causal entries set to -inf, softmax over each row, times V;
// the going-further section fuses the three steps into one kernel so the
// score matrix never reaches HBM. New token i sits at cache row prefix+i and
// sees rows [0, prefix+i].
//
// One workgroup = 4 waves = 64 queries (16 per wave) of one head; grid
// (query tile, head, batch), highest query tiles first (they have the most
// keys). Per 64-key tile:
//   * K rows and V rows are staged in LDS (double-buffered: the global loads
//     of tile t+1 are issued before tile t is computed). K keeps its row
//     layout; V is stored transposed (d-major) so each lane can fetch the 8
//     keys of one d that an MFMA operand needs with two 8-byte LDS reads.
//   * Sᵀ = K·Qᵀ with v_mfma_f32_16x16x32_bf16 (A = K rows, B = this wave's
//     16 queries). Computing the transpose puts each lane on one query and
//     4 keys per 16-key block, which is exactly the operand layout the P·V
//     product needs, so P never leaves registers.
//   * Online softmax in the exp2 domain: scale*log2(e) is applied to the fp32
//     scores; the row max is reduced over the 4 lanes that share a query; the
//     row sum stays per lane until the end. Only tiles that cross the
//     diagonal evaluate the mask; tiles past a wave's last visible key are
//     skipped entirely.
//   * Oᵀ += Vᵀ·Pᵀ with P rounded to bf16 and fp32 accumulation.
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

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int D>
struct Tile {
  static constexpr int SK = D + 8;   // K row stride in LDS (bf16 elements)
  static constexpr int SV = BN + 4;  // Vᵀ row stride in LDS (bf16 elements)
  static constexpr int KCH = BN * D / 8 / kThreads;         // 16B K chunks per thread
  static constexpr int VCH = (BN / 2) * (D / 8) / kThreads; // V row-pair chunks per thread
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");
};

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t *__restrict__ qg, const uint16_t *__restrict__ kg,
    const uint16_t *__restrict__ vg, uint16_t *__restrict__ outg, int Hq,
    int Hkv, int max_length, int Lq, int prefix, float qk_scale,
    int n_qtiles) {
  using T = Tile<D>;
  constexpr int KS = D / 32;   // MFMA k-steps of Q·Kᵀ
  constexpr int NDB = D / 16;  // 16-wide d blocks of the output
  constexpr int NKB = BN / 16; // 16-key blocks per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * T::SK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * T::SV];

  const int qt = n_qtiles - 1 - (int)blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int w = tid / 64;
  const int l = tid % 64;
  const int li = l % 16;  // query within the wave / row within a block
  const int lg = l / 16;  // lane group (k slots 8*lg..8*lg+7)

  const int kv_len = prefix + Lq;
  const int q_end = min((qt + 1) * BM, Lq);
  const int n_tiles = (prefix + q_end + BN - 1) / BN;
  const int qw0 = qt * BM + w * 16;      // first query of this wave
  const int qme = qw0 + li;              // this lane's query
  const bool w_active = qw0 < Lq;
  const int w_kmax = prefix + min(qw0 + 15, Lq - 1);  // last key the wave sees

  const size_t kvbase = ((size_t)b * Hkv + kvh) * (size_t)max_length * D;
  const uint16_t *kbase = kg + kvbase;
  const uint16_t *vbase = vg + kvbase;

  // This lane's query, B operand of Sᵀ = K·Qᵀ (k slots = d).
  bf16x8_t qf[KS];
  {
    const size_t qrow = (((size_t)b * Hq + h) * Lq + (size_t)qme) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qme < Lq)
        v = *reinterpret_cast<const u32x4_t *>(qg + qrow + ks * 32 + 8 * lg);
      qf[ks] = as_bf16x8(v);
    }
  }

  f32x4_t o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;
  float lsum = 0.f;

  // Register staging of one tile's global loads.
  u32x4_t kreg[T::KCH];
  u32x4_t vreg[T::VCH][2];

  auto gload = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j0 + row < kv_len)
        v = *reinterpret_cast<const u32x4_t *>(kbase + (size_t)(j0 + row) * D + col);
      kreg[i] = v;
    }
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
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4_t *>(&Ks[buf][row * T::SK + col]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) {
      const int c = tid + i * kThreads;
      const int col = (c % (D / 8)) * 8;
      const int p = c / (D / 8);  // row pair inside the tile
      const u32x4_t a = vreg[i][0], bb = vreg[i][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // element 2e and 2e+1 of rows 2p and 2p+1, packed (row 2p low half)
        const uint32_t lo = (a[e] & 0xffffu) | (bb[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (bb[e] & 0xffff0000u);
        *reinterpret_cast<uint32_t *>(&Vt[buf][(col + 2 * e) * T::SV + 2 * p]) = lo;
        *reinterpret_cast<uint32_t *>(&Vt[buf][(col + 2 * e + 1) * T::SV + 2 * p]) = hi;
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < n_tiles;
    if (more) gload(t + 1);
    const int j0 = t * BN;
    if (w_active && j0 <= w_kmax) {
      // ---- Sᵀ block scores -------------------------------------------------
      f32x4_t s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t *>(
              &Ks[buf][(kb * 16 + li) * T::SK + ks * 32 + 8 * lg]);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf[ks],
                                                         s[kb], 0, 0, 0);
        }
      }
      // ---- scale, causal mask, row max ----------------------------------------
      const bool diag = j0 + BN - 1 > prefix + qw0;
      const int jlim = prefix + qme;  // last key this query may see
      float mloc = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[kb][r] * qk_scale;
          if (diag && j0 + kb * 16 + 4 * lg + r > jlim) x = kNegInf;
          s[kb][r] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mnew = fmaxf(m, mloc);  // finite: key 0 is always visible
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      // ---- P and Oᵀ += Vᵀ·Pᵀ ------------------------------------------------------
#pragma unroll
      for (int t2 = 0; t2 < BN / 32; ++t2) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(s[2 * t2][r] - mnew);
          p[4 + r] = fast_exp2(s[2 * t2 + 1][r] - mnew);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum += p[e];
        const u32x4_t pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        const bf16x8_t pb = as_bf16x8(pw);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t *vrow = &Vt[buf][(db * 16 + li) * T::SV + 32 * t2 + 4 * lg];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + 16);
          const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), pb,
                                                         o[db], 0, 0, 0);
        }
      }
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- finalise: total row sum over the 4 lanes of a query, divide, store ----
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (qme < Lq) {
    const float inv = 1.f / lsum;
    uint16_t *orow = outg + (((size_t)b * Hq + h) * Lq + (size_t)qme) * D;
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
  dim3 grid(n_qtiles, a.Hq, a.B);
  prefill_kernel<D><<<grid, kThreads, 0, stream>>>(
      static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
      static_cast<const uint16_t *>(a.v), static_cast<uint16_t *>(a.out), a.Hq,
      a.Hkv, a.max_length, a.Lq, a.prefix_len, a.scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace attn
