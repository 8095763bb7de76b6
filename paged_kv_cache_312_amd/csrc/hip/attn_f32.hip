// Paged flash attention in fp32 (the force_fp32 path: "How the Paged KV Cache
// Attention Mechanism Enables Long Sequence Inference in LingBot-Map", section
// "Memory Efficiency Analysis"; fp32 support via force_fp32: "How FlashInfer's
// Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference",
// section "Precision and Hardware Utilization").
//
// Same algorithm and work layout as the bf16 kernel, with fp32 everywhere:
// inputs, v_mfma_f32_32x32x2f32 products, P and the output.  K and V tiles
// are staged row-major in LDS (the fp32 MFMA takes one key per lane half, so V
// needs no transpose).  D = 32 or 64.
#include "attn_common.h"

namespace lbm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
// staging registers of the K/V loads: a native vector (HIP's float4 is a
// struct, whose copies between address spaces keep the staging arrays in
// scratch memory)
typedef float f32x4 __attribute__((ext_vector_type(4)));

// TR: a skip-append step, whose keys [tr_start, kv_len) are the frame's own rows
template <int D, bool TR>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(const BatchArgs b) {
  constexpr int KS = D + 4;          // LDS row strides (floats)
  constexpr int VS = D + 8;
  constexpr int CPR = D / 4;         // 16-byte chunks per key row
  constexpr int KPP = kThreads / CPR;  // keys per loader pass
  constexpr int PASSES = 64 / KPP;
  constexpr int NDB = D / 32;        // 32-column blocks of O^T
  constexpr int HALF = D / 2;        // contraction columns per lane half
  __shared__ __attribute__((aligned(16))) float lds_k[2][64 * KS];
  __shared__ __attribute__((aligned(16))) float lds_v[2][64 * VS];

  int32_t sid;
  const int32_t item = work_item(b, blockIdx.x, sid);
  if (sid < 0) return;
  AttnArgs a = b.s[sid];  // a copy: values, not loads that a memory barrier would repeat
  if (a.desc) {
    a.kv_len = a.desc->kv_len;
    a.n_tiles = a.desc->n_tiles;
    a.tiles_per_split = a.desc->tiles_per_split;
    a.tr_start = a.kv_len;
  }
  const int32_t qt = item % a.n_qt;
  const int32_t grp = item / a.n_qt;
  const int32_t head = grp / a.num_splits;
  const int32_t split = grp - head * a.num_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t HD = a.H * D;
  const int32_t t_begin = split * a.tiles_per_split;
  const int32_t t_end = min(a.n_tiles, t_begin + a.tiles_per_split);
  if (t_end <= t_begin) {
    // a split left without keys (graph-replayed steps keep the capture's split
    // count): an empty partial, weight 0 in the merge
    const int32_t qrow0 = qt * kRowsPerWGf32 + wave * 32 + l32;
    if (qrow0 < a.Tq) {
      const size_t rh = (size_t(split) * a.rows_pad + qrow0) * a.H + head;
      float* po = a.part_o + rh * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(po + db * 32 + 8 * i + 4 * hh) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + rh * 2) = make_float2(-INFINITY, 0.f);
    }
    return;
  }

  // Q as the B operand: row qrow, contraction columns HALF*hh + ks.
  const int32_t qrow = qt * kRowsPerWGf32 + wave * 32 + l32;
  float qf[HALF];
  if (qrow < a.Tq) {
    const float4* qp = reinterpret_cast<const float4*>(
        reinterpret_cast<const float*>(a.q) + size_t(qrow) * HD + head * D + HALF * hh);
#pragma unroll
    for (int i = 0; i < HALF / 4; ++i) {
      const float4 x = qp[i];
      qf[4 * i] = x.x; qf[4 * i + 1] = x.y; qf[4 * i + 2] = x.z; qf[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < HALF; ++i) qf[i] = 0.f;
  }

  const int lc = tid % CPR;
  const int lk = tid / CPR;
  const int32_t col_off = (head * D + lc * 4) * 4;
  f32x4 kreg[PASSES], vreg[PASSES];
  auto load_tile = [&](int32_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const char *kp, *vp;
      const int32_t key = t * 64 + r * KPP + lk;
      kv_rows(a, a.rowtab[key], col_off, kp, vp);
      if (TR && key >= a.tr_start) {
        // the frame's own rows; the padding past kv_len repeats the last one
        // (finite input, whose weights the mask zeroes)
        const size_t off = size_t(min(key, a.kv_len - 1) - a.tr_start) * a.row_bytes + col_off;
        kp = static_cast<const char*>(a.tk) + off;
        vp = static_cast<const char*>(a.tv) + off;
      }
      kreg[r] = *reinterpret_cast<const f32x4*>(kp);
      vreg[r] = *reinterpret_cast<const f32x4*>(vp);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int key = r * KPP + lk;
      *reinterpret_cast<f32x4*>(&lds_k[buf][key * KS + lc * 4]) = kreg[r];
      *reinterpret_cast<f32x4*>(&lds_v[buf][key * VS + lc * 4]) = vreg[r];
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.scale_log2;

  load_tile(t_begin);
  store_tile(0);
  __syncthreads();

  for (int32_t t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile(t + 1);
    const float* K = lds_k[buf];
    const float* V = lds_v[buf];

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
      const float4* kr = reinterpret_cast<const float4*>(K + (kb * 32 + l32) * KS + HALF * hh);
#pragma unroll
      for (int i = 0; i < HALF / 4; ++i) {
        const float4 kx = kr[i];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qf[4 * i + 0], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qf[4 * i + 1], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qf[4 * i + 2], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qf[4 * i + 3], s[kb], 0, 0, 0);
      }
    }
    if ((t + 1) * 64 > a.kv_len) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t key = t * 64 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key >= a.kv_len) s[kb][e] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run)) {
      const float alpha = fast_exp2((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(s[kb][e], c, -mc));
        s[kb][e] = p;
        lsum += p;
      }
    l_run += lsum;

    // O^T[d][row] += sum over keys V[key][d] P[row][key]; one key per lane half
    // per MFMA: element e of s[kb] is key kb*32 + 8(e/4) + 4hh + e%4.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float vv = V[(kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)) * VS + db * 32 + l32];
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[kb][e], o[db], 0, 0, 0);
        }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (a.num_splits == 1) {
    if (qrow < a.Tq) {
      const float inv = 1.f / l_tot;
      float* op = reinterpret_cast<float*>(a.out) + size_t(qrow) * HD + head * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(op + db * 32 + 8 * i + 4 * hh) =
              make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                          o[db][4 * i + 3] * inv);
    }
    return;
  }

  if (qrow < a.Tq) {
    const size_t rh = (size_t(split) * a.rows_pad + qrow) * a.H + head;
    float* po = a.part_o + rh * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(po + db * 32 + 8 * i + 4 * hh) =
            make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
    if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + rh * 2) = make_float2(m_run * c, l_tot);
  }
}

}  // namespace

hipError_t launch_attn_f32(const BatchArgs& b, int32_t head_dim, bool transient, hipStream_t stream) {
  const dim3 grid(8 * b.items_per_xcd), block(kThreads);
  if (head_dim == 64 && transient)
    hipLaunchKernelGGL((attn_f32_kernel<64, true>), grid, block, 0, stream, b);
  else if (head_dim == 64)
    hipLaunchKernelGGL((attn_f32_kernel<64, false>), grid, block, 0, stream, b);
  else if (head_dim == 32 && transient)
    hipLaunchKernelGGL((attn_f32_kernel<32, true>), grid, block, 0, stream, b);
  else if (head_dim == 32)
    hipLaunchKernelGGL((attn_f32_kernel<32, false>), grid, block, 0, stream, b);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int32_t attn_occupancy_f32(int32_t head_dim) {
  int n = 0;
  hipError_t e = head_dim == 32
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<32, false>,
                                                                   kThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<64, false>,
                                                                   kThreads, 0);
  if (e != hipSuccess || n < 1) return 1;
  return n;
}

}  // namespace lbm
