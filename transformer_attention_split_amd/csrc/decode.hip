// Split-KV single-token decode over a static KV cache (gfx950, wave64).
//
// Operation: "MiniCPM4 forward_step Attention Performance Fix", §3 and §4.1 —
// the query of the new token attends only to cache rows [0, position_id]
// (or [0, seq_len) per sequence), and the slice bound replaces the mask, so
// work and bytes read are proportional to the valid length (§2.4 cost table).
//
// Two kernels:
//   decode_split_kernel   grid (split, kv head, batch). One workgroup streams
//       the K and V rows of its split once and serves every query head of the
//       kv group from that single read. Each cache row is read by a group of
//       LPR lanes with one 16-byte load per lane (a wave covers 64/LPR
//       consecutive rows, 1 KiB contiguous); the per-row dot products are
//       reduced with DPP row operations; softmax is the online (running max /
//       running sum) form in the exp2 domain with scale*log2(e) folded into q.
//       The workgroup merges its row groups and writes one partial
//       (max, sum, unnormalised output) per query head.
//   decode_combine_kernel grid (query head, batch). Log-sum-exp merge of the
//       partials of the splits that hold rows, division by the total sum and
//       the cast to the output type.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

template <bool BF16, int VEC>
__device__ __forceinline__ void unpack(const uint4 &w, float (&f)[VEC]) {
  if constexpr (BF16) {
    static_assert(VEC == 8, "bf16 chunk holds 8 values");
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo(x[i]);
      f[2 * i + 1] = bf16hi(x[i]);
    }
  } else {
    static_assert(VEC == 4, "f32 chunk holds 4 values");
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
}

__device__ __forceinline__ int valid_length(const int32_t *seq_lens, int b,
                                            int position_id, int max_length) {
  if (seq_lens == nullptr) return position_id + 1;
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > max_length ? max_length : L);
}

template <bool BF16, int D, int G, int U>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const void *__restrict__ qp, const void *__restrict__ kp,
    const void *__restrict__ vp, const int32_t *__restrict__ seq_lens,
    int position_id, float *__restrict__ ws_ml, float *__restrict__ ws_o,
    int Hq, int Hkv, int max_length, int split_rows, int splits,
    float qscale) {
  constexpr int ELT = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ELT;             // values per 16-byte chunk
  constexpr int LPR = D / VEC;              // lanes per cache row
  constexpr int NG = kDecodeThreads / LPR;  // row groups per workgroup
  constexpr int NW = kDecodeThreads / 64;   // waves per workgroup
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row layout");

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int L = valid_length(seq_lens, b, position_id, max_length);
  const int row0 = s * split_rows;
  if (row0 >= L) return;  // uniform over the workgroup
  const int row1 = min(row0 + split_rows, L);

  const int tid = threadIdx.x;
  const int lr = tid % LPR;   // lane inside the row group
  const int grp = tid / LPR;  // row group

  // Query heads g*G .. g*G+G-1, this lane's VEC dimensions, prescaled.
  float qv[G][VEC];
  {
    const char *qb = static_cast<const char *>(qp) +
                     (((size_t)b * Hq + (size_t)g * G) * D + lr * VEC) * ELT;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 w = *reinterpret_cast<const uint4 *>(qb + (size_t)h * D * ELT);
      unpack<BF16, VEC>(w, qv[h]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[h][e] *= qscale;
    }
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
  constexpr size_t RB = (size_t)D * ELT;  // bytes per cache row
  const char *kb = static_cast<const char *>(kp) + rowbase * RB + lr * 16;
  const char *vb = static_cast<const char *>(vp) + rowbase * RB + lr * 16;

  for (int r = row0 + grp; r < row1; r += NG * U) {
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + u * NG;
      if (rr < row1) {
        kr[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)rr * RB);
        vr[u] = *reinterpret_cast<const uint4 *>(vb + (size_t)rr * RB);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    // Scores (already in the log2 domain through qscale).
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      unpack<BF16, VEC>(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(qv[h][e], kf[e], acc);
        sc[u][h] = group_sum<LPR>(acc);
      }
      if (r + u * NG >= row1) {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[u][h] = kNegInf;
      }
    }
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack<BF16, VEC>(vr[u], vf[u]);
    // Online softmax update, once per U rows.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
      const float mnew = fmaxf(m[h], mx);  // finite: row r is valid
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
        for (int u = 0; u < U; ++u) acc = fmaf(p[u], vf[u][e], acc);
        o[h][e] = acc;
      }
      m[h] = mnew;
    }
  }

  // ---- merge the row groups of the workgroup --------------------------------
  __shared__ float sm_m[NG][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];
  if (lr == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sm_m[grp][h] = m[h];
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = sm_m[0][h];
    for (int i = 1; i < NG; ++i) x = fmaxf(x, sm_m[i][h]);
    M[h] = x;  // finite: at least one group holds a row
    const float w = fast_exp2(m[h] - M[h]);  // 0 for an empty group
    l[h] *= w;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] *= w;
  }
  // Sum over the row groups of a wave (lanes with equal lr).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] += __shfl_xor(o[h][e], off);
    }
  }
  const int wave = tid / 64;
  const int lane = tid % 64;
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_o[wave][h][lr * VEC + e] = o[h][e];
      if (lr == 0) sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;
  for (int i = tid; i < G * D; i += kDecodeThreads) {
    const int h = i / D, d = i % D;
    float x = sm_o[0][h][d];
#pragma unroll
    for (int w = 1; w < NW; ++w) x += sm_o[w][h][d];
    ws_o[((head0 + h) * splits + s) * D + d] = x;
  }
  if (tid < G) {
    float x = sm_l[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) x += sm_l[w][tid];
    float *ml = ws_ml + ((head0 + tid) * splits + s) * 2;
    ml[0] = M[tid];
    ml[1] = x;
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float *__restrict__ ws_ml, const float *__restrict__ ws_o,
    const int32_t *__restrict__ seq_lens, int position_id,
    void *__restrict__ outp, int Hq, int max_length, int split_rows,
    int splits) {
  constexpr int PER = D / 64;  // output values per lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = valid_length(seq_lens, b, position_id, max_length);
  const int n = (L + split_rows - 1) / split_rows;  // splits holding rows
  const size_t head = (size_t)b * Hq + h;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lsum = 1.f;
  if (n > 0) {
    const float *ml = ws_ml + head * splits * 2;
    const float *o = ws_o + head * splits * D + lane * PER;
    float M = ml[0];
    for (int s = 1; s < n; ++s) M = fmaxf(M, ml[2 * s]);
    lsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = fast_exp2(ml[2 * s] - M);
      lsum = fmaf(w, ml[2 * s + 1], lsum);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, o[(size_t)s * D + e], acc[e]);
    }
  }
  if constexpr (BF16) {
    uint16_t *out = static_cast<uint16_t *>(outp) + head * D + lane * PER;
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t *>(out) =
          pack_bf16x2(acc[0] / lsum, acc[1] / lsum);
    } else {
      const uint32_t w = pack_bf16x2(acc[0] / lsum, 0.f);
      out[0] = (uint16_t)(w & 0xffffu);
    }
  } else {
    float *out = static_cast<float *>(outp) + head * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = acc[e] / lsum;
  }
}

template <bool BF16, int D, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
  constexpr int U = 4;
  const float qscale = a.scale * kLog2e;
  dim3 grid1(a.plan.splits, a.Hkv, a.B);
  decode_split_kernel<BF16, D, G, U><<<grid1, kDecodeThreads, 0, stream>>>(
      a.q, a.k, a.v, a.seq_lens, a.position_id, a.ws_ml, a.ws_o, a.Hq, a.Hkv,
      a.max_length, a.plan.split_rows, a.plan.splits, qscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.Hq, a.B);
  decode_combine_kernel<BF16, D><<<grid2, 64, 0, stream>>>(
      a.ws_ml, a.ws_o, a.seq_lens, a.position_id, a.out, a.Hq, a.max_length,
      a.plan.split_rows, a.plan.splits);
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
