// Paged flash attention, 16-bit inputs (bf16 or fp16), MFMA on gfx950 (CDNA4).
//
// Computes, for every query row i and head h of a frame step, softmax over
// the visible keys of q.k / sqrt(D) applied to v, reading K/V straight from
// the patch and special pages through the visible table ("How Paged KV Cache
// Attention Enables ~20 FPS Streaming Inference in LingBot-Map", section
// "FlashInfer Paged-Kernel Integration"; "How the Paged KV Cache Attention
// Mechanism Enables Long Sequence Inference in LingBot-Map", section
// "FlashInfer Kernel Execution").  No mask inside a step.  The pages run the
// kernel natively on either 16-bit type ("How FlashInfer's Paged KV Cache
// Attention Outperforms SDPA Fallback in Streaming Inference", section
// "Precision and Hardware Utilization"): one template, instantiated for bf16
// and fp16, which differ only in the MFMA, the dot product of the row sums
// and the conversions.
//
// Structure (D = 64):
//  * a workgroup = 4 wavefronts = 128 query rows of one head over one key
//    range (split); each wavefront owns 32 rows;
//  * 64-key tiles of K and V go from HBM straight into LDS (row-major, global
//    loads with an LDS destination, no staging registers) through rings of
//    four stages each, one to two tiles ahead of use; one barrier per tile;
//  * the row codes that address those loads travel the same way, a ring of
//    eight tiles' codes in LDS, one stage further ahead, so that waiting for
//    a code never waits for a newer tile;
//  * software pipeline: tile t+1's K Q^T MFMAs start on K operands read during
//    the previous step and are interleaved with tile t's exponentials; tile
//    t+2's K operands are read as soon as they are issued; then tile t's P V
//    MFMAs;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: a lane then holds 16 scores of
//    one query row, so the row max needs one exchange with lane +-32 and the
//    row sum none until the end;
//  * per-step row table (one code per key position) gives each K/V row's
//    address, so the loop does no page arithmetic;
//  * online softmax in fp32 with exp2 and the scale folded in, against a
//    running max that is refreshed (and O rescaled) only when a weight would
//    exceed 256; row sums by 16-bit dot products of the rounded weights;
//  * O^T += V^T P^T on the same MFMA with P taken from registers (no LDS trip),
//    P rounded to the input type (round to nearest even); the V operand comes from the
//    row-major tile through gfx950's LDS transpose reads;
//  * with several splits, each writes (O, m, l) partials that a separate merge
//    kernel combines (a kernel boundary orders them: no fences, which on this
//    chip would write back and invalidate the XCD's L2 that the workgroups
//    share);
//  * one launch may cover several independent streams (a table of per-stream
//    arguments; each workgroup finds its stream), a skip-append step's own
//    rows (the TR instances read them from the caller's buffers), and a
//    graph-replayed step (lengths and tile counts from a step descriptor in
//    the workspace).
#include "attn_common.h"

namespace lbm {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The element type's MFMA (32x32x16, fp32 accumulate) and pair dot product
// (fp32 accumulate).
template <typename T> struct Elt;
template <> struct Elt<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <> struct Elt<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};

constexpr int D = 64;
constexpr int LS = 64;              // LDS row = one key's 64 columns, 128 bytes
constexpr int TILE = 64 * LS;       // elements of one staged K or V tile
constexpr int NST = 4;              // LDS stages of K and of V
constexpr int NCODE = 2 * NST;      // LDS slots of row codes (64 per tile)
// Global loads (all with an LDS destination) each wavefront issues per tile:
// two K, two V, one of row codes.
constexpr int kLoadsPerStep = 5;

// s_waitcnt with only the vector-memory count constrained (expcnt and
// lgkmcnt at their maxima); n < 64.
#define LBM_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// the same, and every LDS read of this wavefront complete (lgkmcnt 0)
#define LBM_WAIT_VMCNT_LDS0(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4))

// Tiles are stored with their 16-byte column chunks XOR-swizzled by row, so
// that the MFMA operand reads hit 64 distinct banks per LDS cycle: the K
// operand reads (16 lanes x 16 B of 16 rows) need 8 distinct chunk positions
// among rows of equal parity; the V transpose reads (32 lanes x 8 B of 4 rows
// and 4 chunks) need rows r and r+2 on opposite halves of the row.
__device__ __forceinline__ int k_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int v_swz(int row) { return ((row >> 1) & 1) * 4; }

// Global load with an LDS destination: every lane reads `bytes` from its own
// address `g`, and the wavefront's data lands contiguously (lane j at byte
// bytes*j) from LDS address `l` (wavefront-uniform).  Issued as inline asm so
// that the compiler neither tracks the LDS write nor adds its own waits for
// it (it cannot tell the ring stages apart and would wait for every such
// load before each LDS read): the kernel orders these loads itself with
// vector-memory waits and barriers.  M0 carries the LDS address; no other
// code in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int bytes>
__device__ __forceinline__ void load_to_lds(const void* g, const void* l) {
  const uint32_t la = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)l)));
  if constexpr (bytes == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_nop 0"
                 :: "s"(la), "v"(g) : "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_nop 0"
                 :: "s"(la), "v"(g) : "m0");
}
#pragma clang diagnostic pop

// 8 keys of V column d for the PV MFMA from a row-major V tile, with two LDS
// transpose reads: within each 16-lane group, source lane s points at
// V[k0 + s/4][d0 + 4(s%4)] and output lane i receives V[k0 .. k0+3][d0 + i].
template <typename V8>
__device__ __forceinline__ V8 v_operand(const uint16_t* p0, const uint16_t* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V8, both);
}

// one kernel per element type: attn_d64_kernel<__bf16> and attn_d64_kernel<_Float16>;
// TR: a skip-append step, whose last keys are the frame's own rows
template <typename T, bool TR>
__global__ __launch_bounds__(kThreads, 2) void attn_d64_kernel(const BatchArgs b) {
  typedef typename Elt<T>::v8 h8;
  typedef typename Elt<T>::v2 h2;
  // Rings indexed by tile position x (x = 0 is the split's first tile): K
  // and V of tile x in stage x mod NST, its row codes in slot x mod NCODE.
  // 66 KB, two workgroups per CU.
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[NST][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[NST][TILE];
  __shared__ __attribute__((aligned(16))) uint32_t lds_code[NCODE][64];

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
    const int32_t qrow0 = qt * 128 + wave * 32 + l32;
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

  // Q as the B operand of S^T = K Q^T: row `qrow`, columns 16ks + 8hh .. +7,
  // pre-multiplied by log2(e)/sqrt(D) (rounded to T) so that the MFMA
  // yields scores in base-2 exponent units.
  const float c = a.scale_log2;
  const int32_t qrow = qt * 128 + wave * 32 + l32;
  h8 qf[4];
  if (qrow < a.Tq) {
    const h8* qp = reinterpret_cast<const h8*>(
        reinterpret_cast<const uint16_t*>(a.q) + size_t(qrow) * HD + head * D + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h8 x = qp[2 * ks];
#pragma unroll
      for (int u = 0; u < 8; ++u) qf[ks][u] = static_cast<T>(static_cast<float>(x[u]) * c);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = h8{};
  }

  // Loads into LDS: a wavefront instruction fills 1 KB = 8 rows of 128 B,
  // lane j writing row j/8, 16-byte slot j%8.  Wavefront w fills rows 8w..8w+7
  // and 32+8w..32+8w+7 of each tile (keys lp and lp+32 for thread tid,
  // lp = tid/8), and slot lc of a row receives the row's chunk lc ^ swizzle,
  // which places the tiles in the swizzled layout the operand reads expect.
  const int lc = tid & 7;
  const int lp = tid >> 3;
  const int32_t k_col = (head * D + ((lc ^ k_swz(lp)) * 8)) * 2;
  const int32_t v_col = (head * D + ((lc ^ v_swz(lp)) * 8)) * 2;
  const int32_t n_t = t_end - t_begin;
  // tile positions past the split's end are clamped to its last tile: such
  // loads land only in stages that are never read again, which keeps the
  // steady-state step free of branches
  auto tile_at = [&](int32_t x) __attribute__((always_inline)) { return t_begin + min(x, n_t - 1); };
  auto row_ptr = [&](uint32_t code, bool v) __attribute__((always_inline)) {
    const bool special = (code >> 31) != 0;
    const char* base = special ? static_cast<const char*>(a.special_pool)
                               : static_cast<const char*>(a.patch_pool);
    const int32_t off = v ? v_col + (special ? a.vstride_special : a.vstride_patch) : k_col;
    return base + (code & 0x7fffffffu) + off;
  };
  // Skip-append step: keys in [tr_start, kv_len) of tile position x come from
  // the frame's own rows (the row table holds position 0's code there, like
  // the padding past kv_len, which keeps its code).  The test is uniform per
  // tile, so tiles of cached keys take the plain path.
  auto own_rows = [&](int32_t x, bool v, const char*& p0, const char*& p1)
                      __attribute__((always_inline)) {
    const int32_t t0 = tile_at(x) * 64;
    if (t0 + 64 > a.tr_start) {
      const char* base = static_cast<const char*>(v ? a.tv : a.tk) + (v ? v_col : k_col);
      const int32_t k0 = t0 + lp, k1 = t0 + lp + 32;
      if (k0 >= a.tr_start && k0 < a.kv_len) p0 = base + size_t(k0 - a.tr_start) * a.row_bytes;
      if (k1 >= a.tr_start && k1 < a.kv_len) p1 = base + size_t(k1 - a.tr_start) * a.row_bytes;
    }
  };
  auto load_k = [&](int32_t stage, uint2 c, int32_t x) __attribute__((always_inline)) {
    const char* p0 = row_ptr(c.x, false);
    const char* p1 = row_ptr(c.y, false);
    if (TR) own_rows(x, false, p0, p1);
    load_to_lds<16>(p0, &lds_k[stage][(8 * wave) * LS]);
    load_to_lds<16>(p1, &lds_k[stage][(32 + 8 * wave) * LS]);
  };
  auto load_v = [&](int32_t stage, uint2 c, int32_t x) __attribute__((always_inline)) {
    const char* p0 = row_ptr(c.x, true);
    const char* p1 = row_ptr(c.y, true);
    if (TR) own_rows(x, true, p0, p1);
    load_to_lds<16>(p0, &lds_v[stage][(8 * wave) * LS]);
    load_to_lds<16>(p1, &lds_v[stage][(32 + 8 * wave) * LS]);
  };
  // all 64 codes of tile position x into their slot (every wavefront loads
  // the whole slice, so each one waits only for its own loads)
  auto load_codes = [&](int32_t x) __attribute__((always_inline)) {
    load_to_lds<4>(a.rowtab + tile_at(x) * 64 + lane, &lds_code[x & (NCODE - 1)][0]);
  };
  auto codes_of = [&](int32_t x) __attribute__((always_inline)) {
    const uint32_t* c = lds_code[x & (NCODE - 1)];
    return make_uint2(c[lp], c[lp + 32]);
  };
  // barrier without a memory fence (the fence would wait for every load
  // into LDS): each use follows an explicit wait for this wavefront's loads
  // into LDS that must have landed and for all its LDS reads, since the
  // compiler may move the consumers of those reads past the barrier
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // K operand: row kb*32 + l32, chunk 2ks + hh (swizzle depends on l32 only).
  // V transpose read: within each 16-lane group g, lane s points at row
  // 4(g/2) + s/4 (+ 16G + 8r) and column db*32 + 16(g%2) + 4(s%4); the row's
  // swizzle is a lane constant, and the column sits in chunk
  // db*4 + 2(g%2) + (s%4)/2, at half (s%2).
  const int k_row = l32 * LS;
  const int k_x = k_swz(l32);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int v_row = (4 * (g16 >> 1) + (s16 >> 2)) * LS;
  const int v_x = v_swz(4 * (g16 >> 1) + (s16 >> 2));
  const int v_c = 2 * (g16 & 1) + ((s16 & 3) >> 1);
  const int v_rd0 = v_row + (((0 * 4 + v_c) ^ v_x) * 8) + 4 * (s16 & 1);
  const int v_rd1 = v_row + (((1 * 4 + v_c) ^ v_x) * 8) + 4 * (s16 & 1);

  // the 8 K operands of a tile (S^T = K Q^T, key blocks kb, column steps ks)
  auto k_reads = [&](const uint16_t* K, h8* kf) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[kb * 4 + ks] = *reinterpret_cast<const h8*>(
            K + k_row + kb * 32 * LS + (((2 * ks + hh) ^ k_x) * 8));
  };
  // the 8 V operands of a tile (O^T = V^T P^T, column blocks db, key groups G)
  auto v_reads = [&](const uint16_t* V, h8* vf) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const uint16_t* p = V + (db == 0 ? v_rd0 : v_rd1) + (16 * G) * LS;
        vf[db * 4 + G] = v_operand<h8>(p, p + 8 * LS);
      }
  };
  // S^T[key][row] - m of one tile, in base-2 units: lane holds row l32 and
  // keys kb*32 + 8i + 4hh + j; the accumulator starts from `neg_m` (every
  // element -m), so the running max is subtracted by the MFMA itself.
  auto qk = [&](const h8* kf, f32x16* s, const f32x16& neg_m) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = Elt<T>::mfma(kf[kb * 4], qf[0], neg_m);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
        s[kb] = Elt<T>::mfma(kf[kb * 4 + ks], qf[ks], s[kb]);
    }
  };

  f32x16 o[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = 0.f;  // running max of this row's scores in base-2 units (stale between jumps)
  float l_run = 0.f;  // this lane's share of the row sum, relative to m_run
  f32x16 neg_m;       // -m_run in every element: the QK accumulator start
#pragma unroll
  for (int e = 0; e < 16; ++e) neg_m[e] = 0.f;
  const h2 ones = {static_cast<T>(1.0f), static_cast<T>(1.0f)};

  // p = 2^(s - shift) in T (s already relative to m_run), grouped as the
  // B operand of the PV MFMA (group G = 2kb + g holds elements 8g..8g+7 of
  // s[kb]); returns this lane's sum of the rounded p (exactly the weights the
  // PV product uses).  shift is 0 except after a refresh of the max.
  auto exponentiate = [&](const f32x16* s, float shift, h8* pb) __attribute__((always_inline)) {
    float lt[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        h8 v;
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = static_cast<T>(fast_exp2(s[kb][8 * g + u] - shift));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const h2 pr = {v[2 * u], v[2 * u + 1]};
          lt[kb] = Elt<T>::dot2(pr, ones, lt[kb]);
        }
        pb[2 * kb + g] = v;
      }
    return lt[0] + lt[1];
  };

  // Prologue: row codes of tile positions 0 .. 2NST-1; K of positions
  // 0 .. NST-1 and V of 0 .. NST-2; then S of position 0.  Step i (below)
  // loads the codes of position i+2NST, reads those of i+NST and loads K of
  // i+NST with them, and V of i+NST-1 with the codes read one step earlier.
#pragma unroll
  for (int x = 0; x < NCODE; ++x) load_codes(x);
  LBM_WAIT_VMCNT(0);
  asm volatile("" ::: "memory");  // the code reads below stay after the wait
  uint2 code_v;
#pragma unroll
  for (int x = 0; x < NST; ++x) {
    code_v = codes_of(x);
    load_k(x, code_v, x);
    if (x < NST - 1) load_v(x, code_v, x);
  }
  // code_v: position NST-1, for the V load of step 0
  LBM_WAIT_VMCNT_LDS0(0);
  barrier();
  f32x16 s_a[2], s_b[2];
  h8 kf[8];  // K operands of the next tile position's K Q^T
  k_reads(lds_k[0], kf);
  qk(kf, s_a, neg_m);
  k_reads(lds_k[1], kf);
  LBM_WAIT_VMCNT_LDS0(63);  // stage 0 of K is reloaded in the first step
  barrier();

  // Softmax against the running max as it stands (the scores arrive with it
  // subtracted); the row max of the tile is taken on the split's first tile
  // and whenever some weight would leave [0, 256] (a jump of the max): then O
  // and l are rescaled and the tile redone.  Any max that is not below the
  // true one gives the same quotient, since numerator and denominator share
  // it; the first tile's refresh makes the largest weight 1, so the row sum
  // never underflows.
  // s_nxt (nullable): the next tile's scores, already issued relative to the
  // old max, are moved to the new one.
  auto refresh_max = [&](const f32x16* s_cur, f32x16* s_nxt, h8* pb, float& lt, bool first)
                         __attribute__((always_inline)) {
    if (__ballot(!(lt <= 256.f)) || first) {
      float mx = s_cur[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s_cur[kb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));  // tile max - m_run
      const float step_up = first ? mx : fmaxf(mx, 0.f);
      const float alpha = first ? 0.f : fast_exp2(-step_up);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      lt = exponentiate(s_cur, step_up, pb);
      m_run += step_up;
#pragma unroll
      for (int e = 0; e < 16; ++e) neg_m[e] = -m_run;
      if (s_nxt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s_nxt[kb][e] -= step_up;
      }
    }
  };
  // O^T[d][row] += V^T[d][keys] P^T[keys][row]
  auto pv = [&](const h8* vf, const h8* pb) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int G = 0; G < 4; ++G)
        o[db] = Elt<T>::mfma(vf[db * 4 + G], pb[G], o[db]);
  };

  // Steady-state step for tile position i (not the split's last): s_cur
  // holds its scores, s_nxt receives position i+1's, whose K operands are
  // already in registers (read during step i-1), so its K Q^T MFMAs start at
  // once and are interleaved with position i's exponentials: the matrix
  // cores run while the vector ALUs work.  The step's loads into LDS (to
  // stages last read in the previous step) and its V operand reads go out
  // first; position i+2's K operands are read once the K Q^T MFMAs have
  // consumed i+1's.  At the end each wavefront waits for its loads of step
  // i-1 (position i+3's K, the next step's V and codes), then the barrier
  // publishes them to the workgroup.
  auto step = [&](int32_t i, f32x16* s_cur, f32x16* s_nxt) __attribute__((always_inline)) {
    const uint2 code_k = codes_of(i + NST);
    load_codes(i + 2 * NST);
    h8 vf[8], pb[4];
    v_reads(lds_v[i & (NST - 1)], vf);
    load_k(i & (NST - 1), code_k, i + NST);
    load_v((i + NST - 1) & (NST - 1), code_v, i + NST - 1);
    qk(kf, s_nxt, neg_m);
    float lt = exponentiate(s_cur, 0.f, pb);
    k_reads(lds_k[(i + 2) & (NST - 1)], kf);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // codes
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // first exponentials
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      if (u == 1) __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // V reads
      if (u == 7) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // next K reads
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // ten VALU
    }
    refresh_max(s_cur, s_nxt, pb, lt, i == 0);
    l_run += lt;
    pv(vf, pb);
    code_v = code_k;
    // this wavefront's reads of the stages refilled next step are complete
    // (the compiler may sink their consumers past the barrier), and its
    // loads of step i-1 have landed
    LBM_WAIT_VMCNT_LDS0(kLoadsPerStep * (NST - 3));
    barrier();
  };
  // The split's last tile: no next tile; keys past the visible set masked.
  auto last_step = [&](int32_t i, f32x16* s_cur) __attribute__((always_inline)) {
    const int32_t t = t_begin + i;
    {
      // element e of s_cur[kb] is key t*64 + 4hh + (kb*32 + 8(e/4) + e%4);
      // applied unconditionally (once per split) to keep one copy of s_cur
      const int32_t lim = a.kv_len - t * 64 - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          s_cur[kb][e] = kb * 32 + 8 * (e >> 2) + (e & 3) >= lim ? -INFINITY : s_cur[kb][e];
    }
    h8 vf[8], pb[4];
    v_reads(lds_v[i & (NST - 1)], vf);
    float lt = exponentiate(s_cur, 0.f, pb);
    refresh_max(s_cur, nullptr, pb, lt, i == 0);
    l_run += lt;
    pv(vf, pb);
  };
  // unrolled by two so that the two score buffers swap roles instead of
  // being copied
  int32_t i = 0;
  for (; i + 2 < n_t; i += 2) {
    step(i, s_a, s_b);
    step(i + 1, s_b, s_a);
  }
  if (n_t - i == 2) {
    step(i, s_a, s_b);
    s_a[0] = s_b[0];  // one inlined copy of the last step
    s_a[1] = s_b[1];
    ++i;
  }
  last_step(i, s_a);

  // loads of clamped positions may still be in flight: the workgroup's LDS
  // must not be released under them
  LBM_WAIT_VMCNT(0);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (a.num_splits == 1) {
    if (qrow < a.Tq) {
      const float inv = 1.f / l_tot;
      T* op = reinterpret_cast<T*>(a.out) + size_t(qrow) * HD + head * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typedef T h4 __attribute__((ext_vector_type(4)));
          h4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = static_cast<T>(o[db][4 * i + j] * inv);
          *reinterpret_cast<h4*>(op + db * 32 + 8 * i + 4 * hh) = w;
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
}

}  // namespace

hipError_t launch_attn16(const BatchArgs& b, int32_t head_dim, bool fp16, bool transient,
                         hipStream_t stream) {
  if (head_dim != 64) return hipErrorInvalidValue;
  const dim3 grid(8 * b.items_per_xcd), block(kThreads);
  if (fp16 && transient)
    hipLaunchKernelGGL((attn_d64_kernel<_Float16, true>), grid, block, 0, stream, b);
  else if (fp16)
    hipLaunchKernelGGL((attn_d64_kernel<_Float16, false>), grid, block, 0, stream, b);
  else if (transient)
    hipLaunchKernelGGL((attn_d64_kernel<__bf16, true>), grid, block, 0, stream, b);
  else
    hipLaunchKernelGGL((attn_d64_kernel<__bf16, false>), grid, block, 0, stream, b);
  return hipGetLastError();
}

int32_t attn_occupancy16() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_d64_kernel<__bf16, false>, kThreads, 0) !=
          hipSuccess ||
      n < 1)
    return 1;
  return n;
}

}  // namespace lbm
