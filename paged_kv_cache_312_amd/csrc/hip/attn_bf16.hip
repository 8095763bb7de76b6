// Paged flash attention, bf16 inputs, MFMA on gfx950 (CDNA4).
//
// Computes, for every query row i and head h of a frame step, softmax over
// the visible keys of q.k / sqrt(D) applied to v, reading K/V straight from
// the patch and special pages through the visible table ("How Paged KV Cache
// Attention Enables ~20 FPS Streaming Inference in LingBot-Map", section
// "FlashInfer Paged-Kernel Integration"; "How the Paged KV Cache Attention
// Mechanism Enables Long Sequence Inference in LingBot-Map", section
// "FlashInfer Kernel Execution").  No mask inside a step.
//
// Structure (D = 64):
//  * a workgroup = 4 wavefronts = 128 query rows of one head over one key
//    range (split); each wavefront owns 32 rows;
//  * per 64-key tile, K is staged in LDS row-major and V transposed (key-major
//    columns, keys permuted so each lane's MFMA operand is one 16-byte read),
//    double-buffered, one barrier per tile; the next tile's global loads are
//    issued before the current tile's math;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a lane then holds 16 scores of
//    one query row, so the row max needs one exchange with lane +-32 and the
//    row sum none until the end;
//  * online softmax in fp32 with exp2 and the scale folded in; O is rescaled
//    only when some row's running max grows;
//  * O^T += V^T P^T on the same MFMA with P taken from registers (no LDS trip),
//    P rounded to bf16 (round to nearest even);
//  * with several splits, each writes (O, m, l) partials and the last
//    workgroup of a (query group, head) merges them.
#include "attn_common.h"

namespace lbm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 64;
constexpr int LS = 72;              // LDS row stride in bf16 elements (64 + 8)
constexpr int TILE = 64 * LS;       // elements of one staged K or V^T tile

// Column of key k (0..63) inside a V^T row: within each 16-key group, lane
// half h reads 8 contiguous columns holding keys {4h..4h+3, 8+4h..8+4h+3}.
__device__ __forceinline__ int vt_col(int k) {
  const int G = k >> 4, kk = k & 15;
  const int a = kk >> 3, h = (kk >> 2) & 1, j = kk & 3;
  return (G << 4) + (h << 3) + (a << 2) + j;
}

__global__ __launch_bounds__(kThreads) void attn_bf16_d64_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE];  // [buffer][K | V^T]

  const int32_t item = work_item(a, blockIdx.x);
  if (item < 0) return;
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

  // Q as the B operand of S^T = K Q^T: row `qrow`, columns 16ks + 8hh .. +7.
  const int32_t qrow = qt * 128 + wave * 32 + l32;
  bf16x8 qf[4];
  if (qrow < a.Tq) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const uint16_t*>(a.q) + size_t(qrow) * HD + head * D + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qp[2 * ks];
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = bf16x8{};
  }

  // Loader: thread -> 16-byte chunk lc of keys 2lp and 2lp+1 of a tile.
  const int lc = tid & 7;
  const int lp = tid >> 3;
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int32_t t) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      int32_t vd;
      const uint16_t* kp = key_row<uint16_t>(a, head, t * 64 + 2 * lp + e, HD, D, vd);
      if (kp) {
        kreg[e] = *reinterpret_cast<const uint4*>(kp + lc * 8);
        vreg[e] = *reinterpret_cast<const uint4*>(kp + vd + lc * 8);
      } else {
        kreg[e] = make_uint4(0, 0, 0, 0);
        vreg[e] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  const int vcol = vt_col(2 * lp);  // even: keys 2lp, 2lp+1 sit in adjacent columns
  auto store_tile = [&](int buf) {
    uint16_t* K = lds[buf][0];
    uint16_t* Vt = lds[buf][1];
    *reinterpret_cast<uint4*>(K + (2 * lp) * LS + lc * 8) = kreg[0];
    *reinterpret_cast<uint4*>(K + (2 * lp + 1) * LS + lc * 8) = kreg[1];
    const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t w0 = v0[m >> 1], w1 = v1[m >> 1];
      const uint32_t packed = (m & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                      : ((w0 & 0xffffu) | (w1 << 16));
      *reinterpret_cast<uint32_t*>(Vt + (lc * 8 + m) * LS + vcol) = packed;
    }
  };

  f32x16 o[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
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
    const uint16_t* K = lds[buf][0];
    const uint16_t* Vt = lds[buf][1];

    // scores: S^T[key][row], lane holds row l32 and keys kb*32 + 8i + 4hh + j
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(K + (kb * 32 + l32) * LS + ks * 16 + hh * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    if ((t + 1) * 64 > a.kv_len) {  // the final tile: keys past the visible set
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
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;

    // P in bf16, grouped as the B operand of the PV MFMA: group G = 2kb + g
    // holds elements 8g..8g+7 of s[kb].
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float p = fast_exp2(fmaf(s[kb][8 * g + u], c, -mc));
          lsum += p;
          pb[2 * kb + g][u] = static_cast<__bf16>(p);
        }
    l_run += lsum;

    // O^T[d][row] += V^T[d][keys] P^T[keys][row]
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(Vt + (db * 32 + l32) * LS + G * 16 + hh * 8);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[G], o[db], 0, 0, 0);
      }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (a.num_splits == 1) {
    if (qrow < a.Tq) {
      const float inv = 1.f / l_tot;
      __bf16* op = reinterpret_cast<__bf16*>(a.out) + size_t(qrow) * HD + head * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = static_cast<__bf16>(o[db][4 * i + j] * inv);
          *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * i + 4 * hh) = w;
        }
    }
    return;
  }

  if (qrow < a.Tq) {
    const size_t rh = (size_t(split) * a.rows_pad + qrow) * a.H + head;
    float* po = a.part_o + rh * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(po + db * 32 + 8 * i + 4 * hh) =
            make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
    if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + rh * 2) = make_float2(m_run, l_tot);
  }
  if (arrive_last(a, qt * a.H + head)) merge_splits<__bf16, D>(a, qt, head);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bf16_d64_kernel, dim3(8 * a.items_per_xcd), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int32_t attn_occupancy_bf16() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_d64_kernel, kThreads, 0) !=
          hipSuccess ||
      n < 1)
    return 1;
  return n;
}

}  // namespace lbm
