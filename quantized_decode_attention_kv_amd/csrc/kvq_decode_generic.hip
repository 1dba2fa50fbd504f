// kv_decode_attn, vector-ALU kernel for gfx950: any supported shape (head widths
// that are multiples of 32 up to 256, 1..16 query heads per KV head, 1/2/3/4/8-bit
// codes, the HeadQ side code).  The matrix-core kernel (kvq_decode_mfma.hip) takes
// the shapes mfma_takes() accepts; this file also holds the dispatcher of both.
//
// Single-token decode attention, out = softmax(scale * q K^T) V, computed
// directly from the packed cache: key x_hat = code * s + z with one (s, z) per
// (key group of k_group tokens, channel), value x_hat = code * s + z with one (s, z) per (token,
// group of v_group = 32, 64 or 128 channels).  The retained fp16 tokens are visited as a separate segment;
// attention does not depend on token order ("LogQuant: Log-Distributed 2-Bit
// Quantization of KV Cache", section 4, A.V = A_P.V_P).  Scores use the scale of
// "HeadQ" section 2.1 / "Thin Keys, Full Values" section 2 (Dk may differ from Dv).
//
// Work split: one workgroup per (partition, kv head, batch row).  The Hq/Hkv query
// heads sharing a kv head are all handled by that workgroup, so each packed byte is
// read from HBM once per decode step.  Within the workgroup each wave owns every
// 4th key group of the partition and keeps its own online-softmax state (running
// max m, running sum l, unnormalised output o); waves are merged through LDS at the
// end, partitions by the merge kernel that follows (kvq_decode_merge.hip).
//
// Dequantization is folded into the dot products so no dequantized tile is ever
// materialised:
//   q . k_hat_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c          (keys, per group)
//   sum_t p_t v_hat_tc = sum_t (p_t s_t,g(c)) code_tc + sum_t p_t z_t,g(c)   (values)
// so the inner loops are one integer extract, one int->float convert and G fused
// multiply-adds per code.
#include <atomic>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"
#include "kvq_rotate.hpp"
#include "kvq_vlayout.hpp"

namespace kvq {

hipError_t launch_merge(const DecodeArgs& a, int parts, hipStream_t stream);

namespace {

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = kDecodeThreads;
constexpr int kMaxVChansPerLane = KVQ_MAX_HEAD_DIM / 64;

__device__ __forceinline__ float sum32(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 32);
  return v;
}
__device__ __forceinline__ float max32(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 32));
  return v;
}
__device__ __forceinline__ float sum64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Online-softmax state of one wave for G queries.  m, l are wave-uniform; o holds
// the lane's value channels c = lane + 64 j.
template <int G>
struct SoftmaxState {
  float m[G], l[G];
  float o[G][kMaxVChansPerLane];
};

// Fold 32 new scores (lane t and t+32 hold the same score of token t; tokens
// beyond the valid count carry -inf) into the state; returns p_t in pv[].
template <int G>
__device__ __forceinline__ void softmax_update(SoftmaxState<G>& st, const float (&s)[G], float (&pv)[G]) {
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float gmax = max32(s[i]);
    const float m_new = fmaxf(st.m[i], gmax);
    // m_new is finite as soon as one real token was seen
    const float alpha = st.m[i] == -INFINITY ? 0.0f : exp2f(st.m[i] - m_new);
    pv[i] = s[i] == -INFINITY ? 0.0f : exp2f(s[i] - m_new);
    const float lsum = sum32(pv[i]);
    st.l[i] = st.l[i] * alpha + lsum;
    st.m[i] = m_new;
#pragma unroll
    for (int j = 0; j < kMaxVChansPerLane; ++j) st.o[i][j] *= alpha;
  }
}

// Dynamic LDS layout (floats):
//   qs   [G][Dk]                   scaled queries, shared by the waves
//   per wave w: kq [Dk][G]          q_c * s_c of the current key group
//               pp [32][ngv][G]     p_t * s_t,g of the current value rows
//               pz [ngv][G]         sum_t p_t * z_t,g
// After the loops the per-wave area is reused for the wave merge.
template <int G>
__host__ __device__ inline int wave_lds_floats(int Dk, int Dv) {
  const int ngv = Dv / KVQ_GROUP;
  return Dk * G + KVQ_GROUP * ngv * G + ngv * G;
}

template <int G, int QDT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs a) {
  extern __shared__ float lds[];
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Dk = a.L.Dk, Dv = a.L.Dv, kb = a.L.k_bits, vb = a.L.v_bits;
  const int vg = a.L.v_group, ngv = Dv / vg;  // value groups per token (the LDS areas are sized for Dv / 32)
  const int ksh = a.L.k_group == 128 ? 2 : (a.L.k_group == 64 ? 1 : 0);  // key group = code groups >> ksh
  const int nG = a.L.n_groups, R = a.L.R, P = a.P;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;

  const int g0 = int(int64_t(p) * nG / P), g1 = int(int64_t(p + 1) * nG / P);
  const int r0 = int(int64_t(p) * R / P), r1 = int(int64_t(p + 1) * R / P);

  float* qs = lds;
  float* wbase = lds + G * Dk + wave * wave_lds_floats<G>(Dk, Dv);
  float* kq = wbase;
  float* pp = kq + Dk * G;
  float* pz = pp + KVQ_GROUP * ngv * G;

  // scaled queries of the G heads sharing this kv head (log2-domain scores)
  for (int i = tid; i < G * Dk; i += kThreads) {
    const int qi = i / Dk, c = i - qi * Dk;
    qs[i] = a.scale * kLog2e * load_q<QDT>(a.q, (int64_t(b) * a.L.Hq + int64_t(h) * G + qi) * Dk + c);
  }
  if (a.L.flags & KVQ_KEY_ROTATION) {
    // the packed keys are rotated: rotate the queries the same way (butterflies in
    // increasing h over LDS, one pass per h), so the scores keep their values
    for (int hh = 1; hh < Dk; hh <<= 1) {
      __syncthreads();
      for (int i = tid; i < G * Dk / 2; i += kThreads) {
        const int lo = (i / hh) * 2 * hh + i % hh;  // rows are Dk wide and Dk is a power of two
        const float u = qs[lo], v = qs[lo + hh];
        qs[lo] = u + v;
        qs[lo + hh] = u - v;
      }
    }
    __syncthreads();
    const float sc = rotation_scale(31 - __builtin_clz(unsigned(Dk)));
    for (int i = tid; i < G * Dk; i += kThreads) qs[i] *= sc;
  }

  // HeadQ side code: pr[i][k] = (U^T q_i)_k in the same scaled units as the scores
  __shared__ float pr[KVQ_MAX_GQA * kMaxSideRank];
  const int rank = a.side_rank;
  if (rank > 0) {
    __syncthreads();  // qs complete
    for (int i = tid; i < G * rank; i += kThreads) {
      const int qi = i / rank, k = i - qi * rank;
      float acc = 0.0f;
      for (int c = 0; c < Dk; ++c) acc = fmaf(qs[qi * Dk + c], a.side_u[(int64_t(h) * Dk + c) * rank + k], acc);
      pr[i] = acc;
    }
  }

  SoftmaxState<G> st;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxVChansPerLane; ++j) st.o[i][j] = 0.0f;
  }
  __syncthreads();

  const int t = lane & 31, hf = lane >> 5;
  const int kw = Dk * kb / 32, kper = 32 / kb;
  const uint32_t kmask = (1u << kb) - 1u, vmask = (1u << vb) - 1u;

  // ------------------------------------------------------------ quantized groups
  const int n_iter = (g1 - g0 + kWaves - 1) / kWaves;
  for (int it = 0; it < n_iter; ++it) {
    const int g = g0 + it * kWaves + wave;
    const bool active = g < g1;
    float bias[G];
    if (active) {
      // q'_c = q_c s_c for this group and the zero-point term sum_c q_c z_c
      const int64_t kgi = slab * (a.g_stride >> ksh) + (g >> ksh);  // key group of code group g
      const uint16_t* ks = static_cast<const uint16_t*>(a.cache.k_scale) + kgi * Dk;
      const uint16_t* kz = static_cast<const uint16_t*>(a.cache.k_zero) + kgi * Dk;
#pragma unroll
      for (int i = 0; i < G; ++i) bias[i] = 0.0f;
      for (int c = lane; c < Dk; c += 64) {
        const float s = h2f(ks[c]), z = h2f(kz[c]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float qv = qs[i * Dk + c];
          kq[c * G + i] = qv * s;
          bias[i] += qv * z;
        }
      }
#pragma unroll
      for (int i = 0; i < G; ++i) bias[i] = sum64(bias[i]);
    }
    __syncthreads();

    float pv[G];
    if (active) {
      // scores: lane (t, hf) takes token t and half the key channels
      const uint32_t* row = static_cast<const uint32_t*>(a.cache.k_codes) + ((slab * a.g_stride + g) * KVQ_GROUP + t) * kw;
      float acc[G];
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = 0.0f;
      // channels [hf Dk / 2, (hf + 1) Dk / 2) in ascending order (a half may start
      // inside a word: at 1 bit a 32-channel row is one word)
      const int c_end = (hf + 1) * (Dk / 2);
      if (kb == 3) {  // a bit stream: a code may straddle two words
        for (int c = hf * (Dk / 2); c < c_end; ++c) {
          const float cf = float(stream_code(row, 3 * c, 3));
          const float* kqc = kq + c * G;
#pragma unroll
          for (int i = 0; i < G; ++i) acc[i] = fmaf(kqc[i], cf, acc[i]);
        }
      }
      for (int c = kb == 3 ? c_end : hf * (Dk / 2); c < c_end;) {
        const int w = c / kper;
        const uint32_t word = row[w];
        const int w_end = min(c_end, (w + 1) * kper);
        for (; c < w_end; ++c) {
          const float cf = float((word >> ((c - w * kper) * kb)) & kmask);
          const float* kqc = kq + c * G;
#pragma unroll
          for (int i = 0; i < G; ++i) acc[i] = fmaf(kqc[i], cf, acc[i]);
        }
      }
      float s[G];
#pragma unroll
      for (int i = 0; i < G; ++i) s[i] = acc[i] + __shfl_xor(acc[i], 32, 64) + bias[i];
      if (rank > 0) {  // logit correction (U^T q) . z_hat of this token
        const int64_t j = (slab * a.g_stride + g) * KVQ_GROUP + t;
        const float zs = h2f(a.side_scale[j]), zz = h2f(a.side_zero[j]);
        for (int k = 0; k < rank; ++k) {
          const float zh = fmaf(float(a.side_codes[j * rank + k]), zs, zz);
#pragma unroll
          for (int i = 0; i < G; ++i) s[i] = fmaf(pr[i * rank + k], zh, s[i]);
        }
      }
      softmax_update<G>(st, s, pv);

      // p_t s_t,g into LDS and the zero-point sums
      const int64_t vblk = (slab * a.g_stride + g) * ngv * KVQ_GROUP;
      const uint16_t* vs = static_cast<const uint16_t*>(a.cache.v_scale) + vblk;
      const uint16_t* vz = static_cast<const uint16_t*>(a.cache.v_zero) + vblk;
      for (int gc = 0; gc < ngv; ++gc) {
        const float s_v = h2f(vs[gc * KVQ_GROUP + t]), z_v = h2f(vz[gc * KVQ_GROUP + t]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (hf == 0) pp[(t * ngv + gc) * G + i] = pv[i] * s_v;
          const float zsum = sum32(pv[i] * z_v);
          if (lane == 0) pz[gc * G + i] = zsum;
        }
      }
    }
    __syncthreads();

    if (active) {
      // values: lane owns channels c = lane + 64 j; codes read from the group's
      // bit stream (layout in kvq_vlayout.hpp)
      const uint32_t* vc = static_cast<const uint32_t*>(a.cache.v_codes) + (slab * a.g_stride + g) * (Dv * vb);
      for (int tt = 0; tt < KVQ_GROUP; ++tt) {
#pragma unroll
        for (int j = 0; j < kMaxVChansPerLane; ++j) {
          const int c = lane + 64 * j;
          if (c < Dv) {
            const int bit = value_bit_position(tt, c, Dv, vb);
            const float cf = float(vb == 3 ? stream_code(vc, bit, 3) : (vc[bit >> 5] >> (bit & 31)) & vmask);
            const float* ppt = pp + (tt * ngv + c / vg) * G;
#pragma unroll
            for (int i = 0; i < G; ++i) st.o[i][j] = fmaf(ppt[i], cf, st.o[i][j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxVChansPerLane; ++j) {
        const int c = lane + 64 * j;
        if (c < Dv) {
#pragma unroll
          for (int i = 0; i < G; ++i) st.o[i][j] += pz[(c / vg) * G + i];
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------- retained fp16 rows
  const int n_rchunks = (r1 - r0 + KVQ_GROUP - 1) / KVQ_GROUP;
  const int n_riter = (n_rchunks + kWaves - 1) / kWaves;
  for (int it = 0; it < n_riter; ++it) {
    const int ck = it * kWaves + wave;
    const int rbeg = r0 + ck * KVQ_GROUP;
    const bool active = ck < n_rchunks;
    if (active) {
      const int r = rbeg + t;
      const bool valid = r < r1;
      float acc[G];
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = 0.0f;
      if (valid) {
        const uint16_t* krow = static_cast<const uint16_t*>(a.cache.k_fp16) + (slab * a.r_stride + r) * Dk;
        for (int c = hf * (Dk / 2); c < (hf + 1) * (Dk / 2); ++c) {
          const float kv = h2f(krow[c]);
#pragma unroll
          for (int i = 0; i < G; ++i) acc[i] = fmaf(qs[i * Dk + c], kv, acc[i]);
        }
      }
      float s[G], pv[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float full = acc[i] + __shfl_xor(acc[i], 32, 64);
        s[i] = valid ? full : -INFINITY;
      }
      softmax_update<G>(st, s, pv);
      if (hf == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) pp[t * G + i] = pv[i];
      }
    }
    __syncthreads();
    if (active) {
      const int nrow = min(KVQ_GROUP, r1 - rbeg);
      for (int tt = 0; tt < nrow; ++tt) {
        const uint16_t* vrow = static_cast<const uint16_t*>(a.cache.v_fp16) + (slab * a.r_stride + rbeg + tt) * Dv;
#pragma unroll
        for (int j = 0; j < kMaxVChansPerLane; ++j) {
          const int c = lane + 64 * j;
          if (c < Dv) {
            const float vv = h2f(vrow[c]);
#pragma unroll
            for (int i = 0; i < G; ++i) st.o[i][j] = fmaf(pp[tt * G + i], vv, st.o[i][j]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- merge the waves
  // per wave: m[G], l[G], o[G][Dv]; the merged result goes to res [G][Dv + 2]
  const int mstride = G * (Dv + 2);
  float* mw = lds + G * Dk + wave * mstride;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      mw[i] = st.m[i];
      mw[G + i] = st.l[i];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxVChansPerLane; ++j) {
    const int c = lane + 64 * j;
    if (c < Dv) {
#pragma unroll
      for (int i = 0; i < G; ++i) mw[2 * G + i * Dv + c] = st.o[i][j];
    }
  }
  __syncthreads();
  const float* m0 = lds + G * Dk;
  float* res = lds + G * Dk + kWaves * mstride;
  for (int idx = tid; idx < G * Dv; idx += kThreads) {
    const int i = idx / Dv, c = idx - i * Dv;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m0[w * mstride + i]);
    float Lsum = 0.0f, O = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float e = lse_weight(m0[w * mstride + i], M);
      Lsum += e * m0[w * mstride + G + i];
      O += e * m0[w * mstride + 2 * G + i * Dv + c];
    }
    res[i * (Dv + 2) + 2 + c] = O;
    if (c == 0) {
      res[i * (Dv + 2)] = M;
      res[i * (Dv + 2) + 1] = Lsum;
    }
  }
  __syncthreads();
  finish_partition(a, G, b, h, p, res);
}

template <int G, int QDT>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int Dk = a.L.Dk, Dv = a.L.Dv;
  const int loop_floats = G * Dk + kWaves * wave_lds_floats<G>(Dk, Dv);
  const int merge_floats = G * Dk + (kWaves + 1) * G * (Dv + 2);
  const size_t lds = size_t(loop_floats > merge_floats ? loop_floats : merge_floats) * sizeof(float);
  const dim3 grid(unsigned(a.P), unsigned(a.L.Hkv), unsigned(a.L.B));
  if (lds > 64 * 1024) {
    // gfx950 has 160 KB of LDS per CU: opt in to more than the default 64 KB, once
    // per device, for the largest head widths (the attribute is an upper bound)
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
    if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
      constexpr int W = KVQ_MAX_HEAD_DIM;
      constexpr int lf = G * W + kWaves * (W * G + KVQ_GROUP * (W / KVQ_GROUP) * G + (W / KVQ_GROUP) * G);
      constexpr int mf = G * W + (kWaves + 1) * G * (W + 2);
      constexpr size_t most = size_t(lf > mf ? lf : mf) * sizeof(float);
      static_assert(most <= 160 * 1024, "LDS budget");
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<G, QDT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(most));
      if (e != hipSuccess) return e;
      if (bit) done.fetch_or(bit, std::memory_order_release);
    }
  }
  if (a.kernel_start || a.kernel_stop)
    return launch_decode_timed(reinterpret_cast<const void*>(&decode_kernel<G, QDT>), grid, dim3(kThreads), lds,
                               stream, a);
  hipLaunchKernelGGL((decode_kernel<G, QDT>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int QDT>
hipError_t launch_q(const DecodeArgs& a, hipStream_t stream) {
  switch (a.L.Hq / a.L.Hkv) {
    case 1: return launch_g<1, QDT>(a, stream);
    case 2: return launch_g<2, QDT>(a, stream);
    case 4: return launch_g<4, QDT>(a, stream);
    case 8: return launch_g<8, QDT>(a, stream);
    case 16: return launch_g<16, QDT>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t plan_decode(const DecodeArgs& a, DecodePlan* plan) {
  // the side-code correction is carried by the vector-ALU kernel only
  if (a.side_rank == 0 && mfma_takes(a.L, a.P)) return mfma_decode(a, nullptr, plan, false);
  plan->kernel = KVQ_KERNEL_VALU;
  plan->units = a.P;
  plan->rows = a.P;
  plan->depth = 0;
  plan->ranks = 0;
  plan->waves = int64_t(a.P) * a.L.Hkv * a.L.B * kWaves;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream, hipEvent_t after_decode) {
  hipError_t e;
  if (plan.kernel == KVQ_KERNEL_MFMA) {
    DecodePlan p = plan;
    e = mfma_decode(a, stream, &p, true);
    if (e == hipSuccess && (p.units != plan.units || p.rows != plan.rows))
      e = hipErrorInvalidValue;  // the device changed since planning
  } else {
    switch (a.q_dtype) {
      case KVQ_F32: e = launch_q<KVQ_F32>(a, stream); break;
      case KVQ_F16: e = launch_q<KVQ_F16>(a, stream); break;
      case KVQ_BF16: e = launch_q<KVQ_BF16>(a, stream); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  if (after_decode && (e = hipEventRecord(after_decode, stream)) != hipSuccess) return e;
  if (plan.rows == 1) return hipSuccess;
  return launch_merge(a, plan.rows, stream);
}

}  // namespace kvq
