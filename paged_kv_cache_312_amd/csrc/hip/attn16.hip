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
//  * a workgroup = 8 wavefronts = up to 512 query rows of one head over one
//    key range (split), one workgroup per CU (two wavefronts per SIMD); each
//    wavefront owns up to 64 rows as two halves of 32, so every K and V
//    operand read from LDS feeds two MFMAs, and each tile loaded into LDS
//    serves all the group's rows.  The step's 32-row halves are dealt evenly
//    to the query groups, whose number the planner chooses with the key
//    ranges (1375 rows: 4 groups of 11, 11, 11 and 10 halves), so the groups
//    that share a key range do equal work and stay in step on its tiles in
//    L2; within a group the halves go to the SIMDs first (a step lasts as
//    long as the busiest SIMD).  A wavefront with one half computes that half
//    only; one without rows only loads and keeps the barriers.  When every
//    group leaves its last wavefront without rows (at most 11 halves a
//    group), that wavefront issues all the tile loads and the others none;
//    otherwise each wavefront loads its 8 rows of every tile.  Wavefronts
//    with two halves, and above them the loading ones, run at raised
//    priority;
//  * 64-key tiles of K and V go from HBM straight into LDS (row-major, global
//    loads with an LDS destination, no staging registers) through rings of
//    four stages each, two tiles ahead of use; one barrier per two tiles;
//  * the row codes that address those loads travel the same way, a ring of
//    eight tiles' codes in LDS, two tiles further ahead, so that waiting for
//    a code never waits for a newer tile;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: a lane then holds 16 scores of
//    one query row per half, so the row max needs one exchange with lane +-32
//    and the row sum none until the end;
//  * per-step row table (one code per key position) gives each K/V row's
//    address, so the loop does no page arithmetic;
//  * online softmax in fp32 with exp2 and the scale folded into Q, against a
//    stale running max: kBase (4) unless a row's first max falls outside a
//    window around it (wide for bf16, narrow for fp16) and raised (O
//    rescaled, the block's scores recomputed from LDS) only when a lane's
//    weights of a key block would sum past a type-dependent limit.  The
//    common path starts the score chains at -kBase (the MFMAs' accumulator
//    input) and takes the exponentials of the scores as they are: no
//    subtraction and no bias work.  A wavefront with some max not kBase
//    ("biased") takes a slower path on every tile that subtracts the
//    difference on the vector ALU and redoes key block 0.  Row sums by 16-bit dot products of the rounded
//    weights;
//  * each tile in two 32-key blocks, in the order K Q^T (block 0), K Q^T
//    (block 1) beside block 0's exponentials, P V (block 0) beside block 1's
//    exponentials, P V (block 1), with the order pinned, so that the vector
//    ALU and the matrix cores of a SIMD work at the same time;
//  * O^T += V^T P^T on the same MFMA with P taken from registers (no LDS trip),
//    P rounded to the input type (round to nearest even); the V operand comes from the
//    row-major tile through gfx950's LDS transpose reads;
//  * at most 256 VGPRs and no scratch, one workgroup (two wavefronts per
//    SIMD) per CU; the steady-state loop takes NST steps per iteration, so
//    LDS operand offsets are constants;
//  * with several splits, each writes its partial (O, m, l in fp32) that a
//    separate merge kernel combines (a kernel boundary orders them: no fences, which on this
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

// The element type's MFMA (32x32x16, fp32 accumulate), pair dot product
// (fp32 accumulate) and the range limits of the weights:
//  kJump: the largest sum of a lane's 16 weights of one key block before the
//    running max is raised (keeps every weight, and P in the input type,
//    finite);
//  [kZeroLo, kZeroHi]: the window of a row's first max (base-2 units, less
//    kBase) in which the running max stays kBase.
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
  static constexpr float kJump = 0x1p64f;
  static constexpr float kZeroLo = -32.f, kZeroHi = 32.f;
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
  // fp16 tops out at 65504: weights stay below 2^12
  static constexpr float kJump = 0x1p12f;
  static constexpr float kZeroLo = -4.f, kZeroHi = 8.f;
};

// The running max a row keeps unless its scores call for another (base-2
// units): the score chains start at -kBase, so the weights 2^(s - kBase) of
// unit-scale logits lie below 1 and seldom cross it.  Weights on both sides
// of 1 flip every exponent bit of the P V operand from one to the next; kept
// below it, the operand's upper exponent bits hold still, and the matrix
// cores switch less.  The chains take it as their accumulator input, so the
// offset costs no instruction.
constexpr float kBase = 4.f;

constexpr int D = 64;
constexpr int LS = 64;              // LDS row = one key's 64 columns, 128 bytes
constexpr int TILE = 64 * LS;       // elements of one staged K or V tile
constexpr int NST = 4;              // LDS stages of K and of V
constexpr int NCODE = 2 * NST;      // LDS slots of row codes (64 per tile)
// tiles whose K and V are loaded ahead of use: two fewer than the stages, so
// that a wavefront one step ahead of another (steps between barriers) never
// reloads a stage the other still reads
constexpr int kLead = NST - 2;
// Global loads (all with an LDS destination) each wavefront issues per tile:
// one K, one V, then one of row codes.
constexpr int kWaves = 8;              // wavefronts per workgroup
constexpr int kThreads16 = 64 * kWaves;
constexpr int kLoadsKV = 2;
constexpr int kLoadsPerStep = kLoadsKV + 1;
constexpr int kLoadsPerStepAll = 8 * kLoadsKV + 1;  // the loading wavefront's (every row)
static_assert(kLead == 2, "the barrier after odd steps waits for the tile two steps ahead");
static_assert(NCODE > 2 * kLead, "a code slot is reloaded only after its read");

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

// The least value of type T that is >= x, as a float (the running max is kept
// on T's grid, so that the score MFMAs can subtract it exactly).
template <typename T>
__device__ __forceinline__ float round_up_to(float x) {
  const T t = static_cast<T>(x);  // nearest
  float y = static_cast<float>(t);
  if (y < x) {  // one unit in the last place towards +inf
    uint16_t bits = __builtin_bit_cast(uint16_t, t);
    bits = y >= 0.f ? uint16_t(bits + 1) : uint16_t(bits - 1);
    y = static_cast<float>(__builtin_bit_cast(T, bits));
  }
  return y;
}

// one kernel per element type: attn_d64_kernel<__bf16> and attn_d64_kernel<_Float16>;
// TR: a skip-append step, whose last keys are the frame's own rows; ONE: every
// query group holds at most 11 halves, and each workgroup's last wavefront
// (then without rows) issues all the tile loads
template <typename T, bool TR, bool ONE>
__global__ __launch_bounds__(kThreads16, 1) void attn_d64_kernel(const BatchArgs b) {
  typedef typename Elt<T>::v8 h8;
  typedef typename Elt<T>::v2 h2;
  // Rings indexed by tile position x (x = 0 is the split's first tile): K
  // and V of tile x in stage x mod NST, its row codes in slot x mod NCODE.
  // 66 KB, one workgroup per CU.
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
  // item -> (query group, head, key range); the groups sharing a key range
  // are consecutive items, so they run side by side on one L2.  A head's
  // key ranges go out last first: the last range holds a skip-append step's
  // own rows, read from the caller's buffers, and dispatched early its
  // workgroups have slack when a launch takes more than one round (a slot
  // whose first workgroup ends late takes no second one).
  const int32_t qt = item % a.n_qt;
  const int32_t grp = item / a.n_qt;
  const int32_t head = grp / a.num_splits;
  const int32_t split = a.num_splits - 1 - (grp - head * a.num_splits);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wavefront-uniform (an SGPR), so the LDS addresses of the loads are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t HD = a.H * D;
  const int32_t t_begin = split * a.tiles_per_split;
  const int32_t t_end = min(a.n_tiles, t_begin + a.tiles_per_split);
  // Rows: the step's ceil(Tq / 32) halves of 32 rows are dealt to the n_qt
  // query groups as evenly as whole halves allow (base or base + 1 each, the
  // larger groups first), so that the groups sharing a key range do equal
  // work and stay in step on its tiles.  Within a group, wavefronts w and
  // w + 4 share SIMD w mod 4 and the workgroup's step time follows its
  // busiest SIMD, so the g halves go to the SIMDs first: c_s to SIMD s, at
  // most L = ceil(g / 4) each, the shortfall 4L - g taken where it leaves
  // the fewest odd counts (a wavefront with one half reads as many operands
  // as one with two).  SIMD s takes halves [S_s, S_s + c_s) of the group
  // (S_s = c_0 + .. + c_(s-1)): wavefront s the first two, wavefront s + 4
  // the rest (nh of them: 2, 1 or 0); this lane's row in half h is
  // qrow0 + 32h.
  const int32_t n_half = (a.Tq + 31) / 32;
  const int32_t base = n_half / a.n_qt, rem = n_half - base * a.n_qt;
  const int32_t g_halves = base + (qt < rem ? 1 : 0);
  int32_t nh, qrow0;
  {
    const int32_t L = (g_halves + 3) / 4, e = 4 * L - g_halves;
    int32_t c[4] = {L, L, L, L};
    if (L % 2 == 0) {
      if (e >= 2) c[3] -= 2;
      if (e % 2) c[e >= 2 ? 2 : 3] -= 1;
    } else {
      for (int k = 0; k < 3; ++k)
        if (k < e) c[3 - k] -= 1;
    }
    const int sm = wave & 3, hi = wave >> 2;
    const int32_t S = (sm > 0 ? c[0] : 0) + (sm > 1 ? c[1] : 0) + (sm > 2 ? c[2] : 0);
    const int32_t cs = sm == 0 ? c[0] : sm == 1 ? c[1] : sm == 2 ? c[2] : c[3];
    nh = __builtin_amdgcn_readfirstlane(min(max(cs - 2 * hi, 0), 2));
    qrow0 = 32 * (base * qt + min(qt, rem) + S + 2 * hi) + l32;
  }
  if (t_end <= t_begin) {
    // a split left without keys (graph-replayed steps keep the capture's split
    // count): an empty partial, weight 0 in the merge
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t qrow = qrow0 + 32 * h;
      if (h < nh && qrow < a.Tq) {
        const size_t rh = (size_t(split) * a.rows_pad + qrow) * a.H + head;
        float* po = a.part_o + rh * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4*>(po + db * 32 + 8 * i + 4 * hh) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + rh * 2) = make_float2(-INFINITY, 0.f);
      }
    }
    return;
  }
  // a wavefront without rows (at most two halves on its SIMD) only loads and
  // keeps the workgroup's barriers
  const bool idle = nh == 0;
  // Loads into LDS (ONE: the launch's groups hold at most 11 halves each, so
  // the dealing leaves every group's last wavefront without rows): the last
  // wavefront issues every row's loads of every tile (and the row codes),
  // and the others none, so that the wavefronts with rows spend no
  // instruction on loads (0.4–1.2% faster in A/B at 4 groups of 10 and 11
  // halves).  Otherwise every wavefront loads its share (its 8 rows of each
  // tile).
  constexpr bool own_share = !ONE;
  const bool all_rows = ONE && wave == kWaves - 1;
  // A SIMD's step lasts as long as its two wavefronts' work; the one with two
  // halves has the longer stream, so its instructions go first when both are
  // ready (0.6% faster in A/B; the other way round, 2.9% slower).  A
  // wavefront without rows issues only its share of the tile loads, which
  // every wavefront waits for at the next barrier: it goes first of all
  // (another 0.6–1.2%).
  if (nh == 2) __builtin_amdgcn_s_setprio(2);
  else if (nh == 0) __builtin_amdgcn_s_setprio(3);

  // Q as the B operand of S^T = K Q^T: half h's row, columns 16ks + 8hh ..
  // +7, pre-multiplied by log2(e)/sqrt(D) (rounded to T) so that the MFMA
  // yields scores in base-2 exponent units.
  const float c = a.scale_log2;
  h8 qf[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int32_t qrow = qrow0 + 32 * h;
    if (h < nh && qrow < a.Tq) {
      const h8* qp = reinterpret_cast<const h8*>(
          reinterpret_cast<const uint16_t*>(a.q) + size_t(qrow) * HD + head * D + 8 * hh);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h8 x = qp[2 * ks];
#pragma unroll
        for (int u = 0; u < 8; ++u) qf[h][ks][u] = static_cast<T>(static_cast<float>(x[u]) * c);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[h][ks] = h8{};
    }
  }

  // Loads into LDS: a wavefront instruction fills 1 KB = 8 rows of 128 B,
  // lane j writing row j/8, 16-byte slot j%8.  Sharing the loads, wavefront w
  // fills rows 8w..8w+7 of each tile (key lp for thread tid, lp = tid/8); the
  // loading wavefront fills all eight row blocks.  Slot lc of a row receives
  // the row's chunk lc ^ swizzle, which places the tiles in the swizzled
  // layout the operand reads expect.
  const int lc = tid & 7;
  const int lp = tid >> 3;
  const int32_t k_col = (head * D + ((lc ^ k_swz(lp)) * 8)) * 2;
  const int32_t v_col = (head * D + ((lc ^ v_swz(lp)) * 8)) * 2;
  const int32_t n_t = t_end - t_begin;
  // tile positions past the split's end are clamped to its last tile: such
  // loads land only in stages that are never read again, which keeps the
  // steady-state step free of branches
  auto tile_at = [&](int32_t x) __attribute__((always_inline)) { return t_begin + min(x, n_t - 1); };
  // this lane's column of a K or V row in either pool, as lane constants in
  // VGPRs: a row address is then one select of a base and one add per load
  const char* col_base[2][2] = {
      {static_cast<const char*>(a.patch_pool) + k_col,
       static_cast<const char*>(a.patch_pool) + v_col + a.vstride_patch},
      {static_cast<const char*>(a.special_pool) + k_col,
       static_cast<const char*>(a.special_pool) + v_col + a.vstride_special}};
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) asm volatile("" : "+v"(col_base[p][kv]));
  auto row_ptr = [&](uint32_t code, bool v) __attribute__((always_inline)) {
    const bool special = (code >> 31) != 0;
    const char* base = special ? col_base[1][v] : col_base[0][v];
    return base + (code & 0x7fffffffu);
  };
  // K and V of tile position x into stage x mod NST.  Skip-append step: keys
  // in [tr_start, kv_len) come from the frame's own rows
  // (the row table holds position 0's code there), and so does the padding
  // past kv_len; the test is uniform per tile, and only the step's last tiles
  // take that branch.  tr_c: whether the test is made (steps that load no
  // own row leave it out).
  const std::integral_constant<bool, TR> tr{};
  auto load_kv = [&](auto tr_c, int32_t x, uint32_t c) __attribute__((always_inline)) {
    const int32_t stage = x & (NST - 1);
    const char* k0 = row_ptr(c, false);
    const char* v0 = row_ptr(c, true);
    const int32_t t0 = tile_at(x) * 64;
    if (decltype(tr_c)::value && t0 + 64 > a.tr_start) {
      const char* tk = static_cast<const char*>(a.tk) + k_col;
      const char* tv = static_cast<const char*>(a.tv) + v_col;
      // the padding past kv_len repeats the last own row (finite input, whose
      // weights the mask zeroes; a pool row there may be unwritten memory
      // when every key of the step is the frame's own)
      const int32_t j0 = t0 + lp - a.tr_start;
      const int32_t n_own = a.kv_len - a.tr_start;
      if (j0 >= 0) {
        const int32_t j = min(j0, n_own - 1);
        k0 = tk + size_t(j) * a.row_bytes;
        v0 = tv + size_t(j) * a.row_bytes;
      }
    }
    load_to_lds<16>(k0, &lds_k[stage][(8 * wave) * LS]);
    load_to_lds<16>(v0, &lds_v[stage][(8 * wave) * LS]);
  };
  // all 64 codes of tile position x into their slot (every wavefront loads
  // the whole slice, so each one waits only for its own loads)
  auto load_codes = [&](int32_t x) __attribute__((always_inline)) {
    load_to_lds<4>(a.rowtab + tile_at(x) * 64 + lane, &lds_code[x & (NCODE - 1)][0]);
  };
  auto codes_of = [&](int32_t x) __attribute__((always_inline)) {
    return lds_code[x & (NCODE - 1)][lp];
  };
  // The loading wavefront (the last one, so its 8-row share is rows 56..63,
  // whose K swizzle is the odd row blocks'): rows 8m + l/8, m = 0..7, of
  // position x, from their codes c8[m]; the even row blocks' K chunks sit
  // dk_even bytes from the odd ones' (the V swizzle is the same for all).
  const int32_t dk_even = (head * D + ((lc ^ k_swz(lane >> 3)) * 8)) * 2 - k_col;
  auto load_kv_all = [&](auto tr_c, int32_t x, const uint32_t* c8) __attribute__((always_inline)) {
    const int32_t stage = x & (NST - 1);
    const int32_t t0 = tile_at(x) * 64;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int32_t dk = (m & 1) ? 0 : dk_even;
      const char* k0 = row_ptr(c8[m], false) + dk;
      const char* v0 = row_ptr(c8[m], true);
      if (decltype(tr_c)::value && t0 + 64 > a.tr_start) {
        const int32_t j0 = t0 + 8 * m + (lane >> 3) - a.tr_start;
        const int32_t n_own = a.kv_len - a.tr_start;
        if (j0 >= 0) {
          const int32_t j = min(j0, n_own - 1);
          k0 = static_cast<const char*>(a.tk) + k_col + dk + size_t(j) * a.row_bytes;
          v0 = static_cast<const char*>(a.tv) + v_col + size_t(j) * a.row_bytes;
        }
      }
      load_to_lds<16>(k0, &lds_k[stage][(8 * m) * LS]);
      load_to_lds<16>(v0, &lds_v[stage][(8 * m) * LS]);
    }
  };
  auto codes_of_all = [&](int32_t x, uint32_t* c8) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c8[m] = lds_code[x & (NCODE - 1)][8 * m + (lane >> 3)];
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
  // Step i's loads: K and V of position i+kLead (into the stage read in step
  // i-2, with the codes read at the end of step i-1) and the codes of
  // position i+2kLead.  At the end of step i the wavefront reads the codes
  // of position i+1+kLead (loaded in step i-1), after waiting for them.
  uint32_t code_nx;  // code of this thread's row of the position the next step loads
  auto step_loads = [&](int32_t i, auto tr_c) __attribute__((always_inline)) {
    load_kv(tr_c, i + kLead, code_nx);
    load_codes(i + 2 * kLead);
  };
  // A barrier after odd steps only: before it every wavefront waits for the
  // K and V it loaded this step (position i+2), so that steps i+1 and i+2
  // both find their tiles whole; between barriers a wavefront runs at most
  // one step ahead of another, and its loads go to the stage read two steps
  // earlier (every wavefront finished that step before the last barrier).
  // After even steps the wait only covers the codes read here.  `odd` is a
  // constant in the unrolled loop.
  auto end_step = [&](int32_t i, bool odd) __attribute__((always_inline)) {
    if (odd)
      LBM_WAIT_VMCNT_LDS0(1);
    else
      LBM_WAIT_VMCNT_LDS0(kLoadsPerStep);
    asm volatile("" ::: "memory");  // the code reads below stay after the wait
    if (own_share) code_nx = codes_of(i + 1 + kLead);
    if (odd) barrier();
  };
  // the same for the loading wavefront: every row's codes and loads
  uint32_t code8[8];
  auto step_loads_all = [&](int32_t i, auto tr_c) __attribute__((always_inline)) {
    load_kv_all(tr_c, i + kLead, code8);
    load_codes(i + 2 * kLead);
  };
  auto end_step_all = [&](int32_t i, bool odd) __attribute__((always_inline)) {
    if (odd)
      LBM_WAIT_VMCNT_LDS0(1);
    else
      LBM_WAIT_VMCNT_LDS0(kLoadsPerStepAll);
    asm volatile("" ::: "memory");  // the code reads below stay after the wait
    codes_of_all(i + 1 + kLead, code8);
    if (odd) barrier();
  };
  // the first step whose tile holds own rows (skip-append step)
  const int32_t own_i0 = a.tr_start / 64 - t_begin;

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

  f32x16 o[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[h][db][e] = 0.f;
  // per half: running max of the row's scores in base-2 units (kBase until
  // the row needs another, stale between jumps) and this lane's share of the
  // row sum relative to it
  float m_run[2] = {kBase, kBase};
  float l_run[2] = {0.f, 0.f};
  // some half's running max is not kBase (wavefront-uniform): every tile
  // then takes the rare path, which subtracts the difference from the scores
  int32_t biased = 0;
  const h2 ones = {static_cast<T>(1.0f), static_cast<T>(1.0f)};
  // the score chains' start: -kBase in every element, held in 16 VGPRs for
  // the whole kernel (the empty asm makes it a register value: as a constant
  // shared by a step's four chain starts the compiler would keep it in 16
  // scalar registers and copy it with eight 64-bit moves per step)
  f32x16 c_start = {-kBase, -kBase, -kBase, -kBase, -kBase, -kBase, -kBase, -kBase,
                    -kBase, -kBase, -kBase, -kBase, -kBase, -kBase, -kBase, -kBase};
  asm volatile("" : "+v"(c_start));

  // S^T[key][row] - m of key block kb (keys 32kb .. 32kb+31) of a tile, for
  // the wavefront's NH halves, in base-2 units: lane holds row l32 (+32h) and
  // keys 32kb + 8j + 4hh + u (element 4j + u of s[h][kb]); each K operand
  // read feeds every half's MFMA.  Each chain starts from -kBase; a biased
  // wavefront then subtracts m_run - kBase on the vector ALU.
  auto unbias = [&](auto b_c, auto nh_c, int kb, f32x16 (*s)[2]) __attribute__((always_inline)) {
    if constexpr (decltype(b_c)::value) {
#pragma unroll
      for (int h = 0; h < decltype(nh_c)::value; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[h][kb][e] -= m_run[h] - kBase;
    }
  };
  auto qk_block = [&](auto b_c, auto nh_c, const uint16_t* K, int kb, f32x16 (*s)[2])
                      __attribute__((always_inline)) {
    constexpr int NH = decltype(nh_c)::value;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h8 kf = *reinterpret_cast<const h8*>(K + k_row + kb * 32 * LS +
                                                 (((2 * ks + hh) ^ k_x) * 8));
#pragma unroll
      for (int h = 0; h < NH; ++h)
        s[h][kb] = Elt<T>::mfma(kf, qf[h][ks], ks == 0 ? c_start : s[h][kb]);
    }
    unbias(b_c, nh_c, kb, s);
  };
  // block kb's K operands (4 contraction steps) from stage K
  auto read_k = [&](const uint16_t* K, int kb, h8* kf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[ks] = *reinterpret_cast<const h8*>(K + k_row + kb * 32 * LS + (((2 * ks + hh) ^ k_x) * 8));
  };
  // block 0's score chains from operands read ahead (no bias)
  auto qk_block_kf = [&](auto nh_c, const h8* kf, f32x16 (*s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int h = 0; h < decltype(nh_c)::value; ++h)
        s[h][0] = Elt<T>::mfma(kf[ks], qf[h][ks], ks == 0 ? c_start : s[h][0]);
  };
  // the same with the bias taken at run time (the rare paths)
  auto qk_block_any = [&](auto nh_c, const uint16_t* K, int kb, f32x16 (*s)[2])
                          __attribute__((always_inline)) {
    if (__builtin_amdgcn_readfirstlane(biased))
      qk_block(std::true_type{}, nh_c, K, kb, s);
    else
      qk_block(std::false_type{}, nh_c, K, kb, s);
  };
  // on the split's last tile, keys of block kb past the visible set
  auto mask_block = [&](auto nh_c, int32_t i, int kb, f32x16 (*s)[2]) __attribute__((always_inline)) {
    constexpr int NH = decltype(nh_c)::value;
    const int32_t lim = a.kv_len - (t_begin + i) * 64 - 4 * hh;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s[h][kb][e] = kb * 32 + 8 * (e >> 2) + (e & 3) >= lim ? -INFINITY : s[h][kb][e];
  };
  // Weights are kept as packed pairs of T (one 32-bit word each), so that each
  // pair is rounded once and that one value feeds both the row sum and the
  // PV operand.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  auto pair_of = [&](float a, float b) __attribute__((always_inline)) {
    return __builtin_convertvector((f32x2{a, b}), h2);  // round to nearest even
  };
  // p = 2^(s - shift[h]) of key block kb in T, grouped as the B operand of the
  // PV MFMA (group G = 2kb + g holds elements 8g..8g+7 of s[h][kb]); lt[h]
  // receives this lane's sum of the rounded p (exactly the weights the PV
  // product uses)
  auto exp_block = [&](auto nh_c, const f32x16 (*s)[2], int kb, const float* shift, u32x4 (*pb)[4],
                       float* lt) __attribute__((always_inline)) {
    constexpr int NH = decltype(nh_c)::value;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      lt[h] = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const h2 pr = pair_of(fast_exp2(s[h][kb][8 * g + 2 * u] - shift[h]),
                                fast_exp2(s[h][kb][8 * g + 2 * u + 1] - shift[h]));
          lt[h] = Elt<T>::dot2(pr, ones, lt[h]);
          pb[h][2 * kb + g][u] = __builtin_bit_cast(uint32_t, pr);
        }
      }
    }
  };
  // four of exp_block's weights: elements 4q .. 4q+3 of s[h][kb], added to lt
  auto exp_part = [&](const f32x16 (*s)[2], int h, int kb, int q, u32x4 (*pb)[4], float* lt)
                      __attribute__((always_inline)) {
    u32x4& v = pb[h][2 * kb + (q >> 1)];
    const int o2 = 2 * (q & 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const h2 pr = pair_of(fast_exp2(s[h][kb][4 * q + 2 * u]), fast_exp2(s[h][kb][4 * q + 2 * u + 1]));
      lt[h] = Elt<T>::dot2(pr, ones, lt[h]);
      v[o2 + u] = __builtin_bit_cast(uint32_t, pr);
    }
  };
  auto as_h8 = [&](const u32x4& w) __attribute__((always_inline)) { return __builtin_bit_cast(h8, w); };
  // O^T[d][row] += V^T[d][keys] P^T[keys][row] over key block kb; each V
  // operand read feeds every half's MFMA
  auto pv_block = [&](auto nh_c, const uint16_t* V, int kb, const u32x4 (*pb)[4]) __attribute__((always_inline)) {
    constexpr int NH = decltype(nh_c)::value;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int G = 2 * kb; G < 2 * kb + 2; ++G) {
        const uint16_t* p = V + (db == 0 ? v_rd0 : v_rd1) + (16 * G) * LS;
        const h8 vf = v_operand<h8>(p, p + 8 * LS);
#pragma unroll
        for (int h = 0; h < NH; ++h) o[h][db] = Elt<T>::mfma(vf, as_h8(pb[h][G]), o[h][db]);
      }
  };
  // the row's max over key blocks kb0 .. kb1 minus m_run (both lanes of the
  // row agree)
  auto row_max = [&](const f32x16* s, int kb0, int kb1) __attribute__((always_inline)) {
    float mx = s[kb0][0];
    for (int kb = kb0; kb <= kb1; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // raise half h's running max by at least step_up (>= 0), to the next value
  // on T's grid; step_up receives the raise taken.  O and l scale by
  // 2^-step_up.
  auto raise_max = [&](int h, float& step_up) __attribute__((always_inline)) {
    const float m_new = round_up_to<T>(m_run[h] + step_up);
    step_up = m_new - m_run[h];  // exact: both on T's grid
    const float alpha = fast_exp2(-step_up);
    l_run[h] *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[h][db][e] *= alpha;
    m_run[h] = m_new;
  };
  // One tile: scores, weights, and O += P V for the wavefront's NH halves,
  // by key block so that each block's exponentials run beside the other
  // block's MFMAs: K Q^T of block 0; K Q^T of block 1 beside block 0's
  // weights; P V of block 0 beside block 1's weights; P V of block 1.
  // Softmax runs against the running max as it stands (the scores arrive
  // with it subtracted).  On the split's first tile a row whose max lies
  // outside [kZeroLo, kZeroHi] of kBase takes that max (so the largest
  // weight is 1 and the row sum never underflows); others keep kBase.
  // Afterwards the max is
  // raised only when some lane's weights of a block would sum past kJump (a
  // jump of the max): then the block's scores are recomputed from the stage
  // (resident until the step's barrier), O and l rescaled and the block's
  // weights redone (a jump in block 0 also shifts block 1's scores; one in
  // block 1 finds block 0's terms already in O, which the rescale carries to
  // the new max).  Any max not below the true one gives the same quotient,
  // since numerator and denominator share it.
  auto tile = [&](auto nh_c, int32_t i, bool first, bool last, int stage,
                  const h8* kf0 = nullptr) __attribute__((always_inline)) {
    constexpr int NH = decltype(nh_c)::value;
    const uint16_t* K = lds_k[stage];
    const uint16_t* V = lds_v[stage];
    f32x16 s[2][2];
    u32x4 pb[2][4];
    float lt0[2], lt1[2];
    // scores against a running max of kBase (the rare path below corrects a
    // biased wavefront's)
    if (kf0)
      qk_block_kf(nh_c, kf0, s);
    else
      qk_block(std::false_type{}, nh_c, K, 0, s);
    if (last) mask_block(nh_c, i, 0, s);
    if (first) {
      // the split's first tile (the running max is kBase here)
      qk_block(std::false_type{}, nh_c, K, 1, s);
      if (last) mask_block(nh_c, i, 1, s);
      float r[2];
      bool out[2];
      bool any = false;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        r[h] = row_max(s[h], 0, 1);
        out[h] = !(r[h] >= Elt<T>::kZeroLo && r[h] <= Elt<T>::kZeroHi);
        any = any || out[h];
      }
      if (__ballot(any)) {
#pragma unroll
        for (int h = 0; h < NH; ++h) m_run[h] = out[h] ? round_up_to<T>(r[h] + kBase) : kBase;
        biased = 1;
      }
      float sh[2];
#pragma unroll
      for (int h = 0; h < NH; ++h) sh[h] = m_run[h] - kBase;
      exp_block(nh_c, s, 0, sh, pb, lt0);
      exp_block(nh_c, s, 1, sh, pb, lt1);
#pragma unroll
      for (int h = 0; h < NH; ++h) l_run[h] += lt0[h] + lt1[h];
      pv_block(nh_c, V, 0, pb);
      pv_block(nh_c, V, 1, pb);
      return;
    }
    // block 1's K Q^T MFMAs, each followed by four of block 0's weights
    // (the fences pin the order, so the vector ALU works while the matrix
    // cores do)
    h8 kf1[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf1[ks] = *reinterpret_cast<const h8*>(K + k_row + 32 * LS + (((2 * ks + hh) ^ k_x) * 8));
    lt0[0] = lt0[1] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 4 * NH; ++st) {
      const int ks = st / NH, h = st % NH;
      s[h][1] = Elt<T>::mfma(kf1[ks], qf[h][ks], ks == 0 ? c_start : s[h][1]);
      exp_part(s, st >> 2, 0, st & 3, pb, lt0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last) mask_block(nh_c, i, 1, s);
    bool jump = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) jump = jump || !(lt0[h] <= Elt<T>::kJump);
    const bool rare = __ballot(jump) != 0 || __builtin_amdgcn_readfirstlane(biased) != 0;
    if (__builtin_expect(rare, 0)) {
      // a jump in block 0, or a biased wavefront: both blocks' scores
      // against the running max, then block 0's weights redone against the
      // raised one
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[h][1][e] -= m_run[h] - kBase;
      qk_block_any(nh_c, K, 0, s);
      if (last) mask_block(nh_c, i, 0, s);
      float su[2];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        su[h] = fmaxf(row_max(s[h], 0, 0), 0.f);
        raise_max(h, su[h]);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[h][1][e] -= su[h];
      }
      biased = 1;
      exp_block(nh_c, s, 0, su, pb, lt0);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) l_run[h] += lt0[h];
    // block 0's P V MFMAs, each after four of block 1's weights
    h8 vf0[4];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        const uint16_t* p = V + (db == 0 ? v_rd0 : v_rd1) + (16 * G) * LS;
        vf0[2 * db + G] = v_operand<h8>(p, p + 8 * LS);
      }
    lt1[0] = lt1[1] = 0.f;
#pragma unroll
    for (int st = 0; st < 4 * NH; ++st) {
      const int mi = st / NH, h = st % NH;
      const int db = mi >> 1, G = mi & 1;
      exp_part(s, st >> 2, 1, st & 3, pb, lt1);
      o[h][db] = Elt<T>::mfma(vf0[2 * db + G], as_h8(pb[h][G]), o[h][db]);
      __builtin_amdgcn_sched_barrier(0);
    }
    jump = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) jump = jump || !(lt1[h] <= Elt<T>::kJump);
    if (__ballot(jump)) {
      qk_block_any(nh_c, K, 1, s);
      if (last) mask_block(nh_c, i, 1, s);
      float su[2];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        su[h] = fmaxf(row_max(s[h], 1, 1), 0.f);
        raise_max(h, su[h]);
      }
      biased = 1;
      exp_block(nh_c, s, 1, su, pb, lt1);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) l_run[h] += lt1[h];
    pv_block(nh_c, V, 1, pb);
  };
  // Prologue: row codes of positions 0 .. 2kLead-1, then K and V of
  // positions 0 .. kLead-1, all resident before the first step (steps 0 and 1
  // run before the first barrier).
  if (own_share || all_rows) {
#pragma unroll
    for (int x = 0; x < 2 * kLead; ++x) load_codes(x);
  }
  LBM_WAIT_VMCNT(0);
  asm volatile("" ::: "memory");  // the code reads below stay after the wait
  if (all_rows) {
#pragma unroll
    for (int x = 0; x < kLead; ++x) {
      codes_of_all(x, code8);
      load_kv_all(tr, x, code8);
    }
  } else if (own_share) {
#pragma unroll
    for (int x = 0; x < kLead; ++x) load_kv(tr, x, codes_of(x));
  }
  LBM_WAIT_VMCNT_LDS0(0);
  barrier();
  if (all_rows) codes_of_all(kLead, code8);
  if (own_share) code_nx = codes_of(kLead);

  // Steps before n_plain - 1 load no own row (kLead ahead): they take the
  // loads without the test for it.
  const int32_t n_plain = !TR || own_i0 >= n_t ? n_t : max(own_i0 - kLead + 1, 0);
  // The same barriers on every wavefront: one after the prologue and one
  // after each odd step but the last.
  if (idle) {
    int32_t i = 0;
    if (all_rows) {
      for (; i + 1 < n_plain; ++i) {
        step_loads_all(i, std::false_type{});
        end_step_all(i, (i & 1) != 0);
      }
      for (; i + 1 < n_t; ++i) {
        step_loads_all(i, tr);
        end_step_all(i, (i & 1) != 0);
      }
    } else if (own_share) {
      for (; i + 1 < n_plain; ++i) {
        step_loads(i, std::false_type{});
        end_step(i, (i & 1) != 0);
      }
      for (; i + 1 < n_t; ++i) {
        step_loads(i, tr);
        end_step(i, (i & 1) != 0);
      }
    } else {
      for (; i + 1 < n_t; ++i) end_step(i, (i & 1) != 0);
    }
    LBM_WAIT_VMCNT(0);
    return;
  }
  // NH halves hold rows: a wavefront with one half runs that half only
  auto steps = [&](auto nh_c) __attribute__((always_inline)) {
    if (n_t == 1) {
      tile(nh_c, 0, true, true, 0);
      return;
    }
    if (own_share) step_loads(0, tr);
    tile(nh_c, 0, true, false, 0);
    end_step(0, false);
    // NST steps per iteration, so that each tile's stage (i mod NST, with
    // i = 1 mod NST at the top) is a constant and its LDS operand addresses
    // fold into the instructions' offsets
    int32_t i = 1;
    // each step reads block 0's K operands before issuing its loads, so that
    // their LDS latency overlaps the load addresses.  Two copies on a
    // skip-append step: the steps before the own rows (no test in the loads)
    // and the rest.
    h8 kf0[4];
    auto fast_steps = [&](auto tr_c, int32_t n) __attribute__((always_inline)) {
      for (; i + NST < n; i += NST) {
#pragma unroll
        for (int k = 0; k < NST; ++k) {
          constexpr int kStage0 = 1;  // i = 1 mod NST here
          const int st = (kStage0 + k) & (NST - 1);
          read_k(lds_k[st], 0, kf0);
          __builtin_amdgcn_sched_barrier(0);
          if (own_share) step_loads(i + k, tr_c);
          tile(nh_c, i + k, false, false, st, kf0);
          end_step(i + k, (st & 1) != 0);
        }
      }
    };
    fast_steps(std::false_type{}, n_plain);
    if (TR) fast_steps(tr, n_t);
    for (; i + 1 < n_t; ++i) {
      if (own_share) step_loads(i, tr);
      tile(nh_c, i, false, false, i & (NST - 1));
      end_step(i, (i & 1) != 0);
    }
    tile(nh_c, n_t - 1, false, true, (n_t - 1) & (NST - 1));
  };
  if (nh == 1)
    steps(std::integral_constant<int, 1>{});
  else
    steps(std::integral_constant<int, 2>{});

  // loads of clamped positions may still be in flight: the workgroup's LDS
  // must not be released under them
  LBM_WAIT_VMCNT(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int32_t qrow = qrow0 + 32 * h;
    if (h >= nh || qrow >= a.Tq) continue;
    const float l_tot = l_run[h] + __shfl_xor(l_run[h], 32);
    if (a.num_splits == 1) {
      // the output, rounded once to T
      const float inv = 1.f / l_tot;
      T* op = reinterpret_cast<T*>(a.out) + size_t(qrow) * HD + head * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typedef T h4 __attribute__((ext_vector_type(4)));
          h4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = static_cast<T>(o[h][db][4 * i + j] * inv);
          *reinterpret_cast<h4*>(op + db * 32 + 8 * i + 4 * hh) = w;
        }
    } else {
      // the split's partial: O unnormalised in fp32 beside (m, l) (an output
      // near V's own values, rounded to T here and again after the merge,
      // would carry two roundings of up to half an ulp of T each)
      const size_t rh = (size_t(split) * a.rows_pad + qrow) * a.H + head;
      float* po = a.part_o + rh * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(po + db * 32 + 8 * i + 4 * hh) =
              make_float4(o[h][db][4 * i], o[h][db][4 * i + 1], o[h][db][4 * i + 2],
                          o[h][db][4 * i + 3]);
      if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + rh * 2) = make_float2(m_run[h], l_tot);
    }
  }
}

}  // namespace

template <typename T>
static void launch_inst(const BatchArgs& b, bool one, dim3 grid, dim3 block, hipStream_t stream) {
  if (one)
    hipLaunchKernelGGL((attn_d64_kernel<T, false, true>), grid, block, 0, stream, b);
  else
    hipLaunchKernelGGL((attn_d64_kernel<T, false, false>), grid, block, 0, stream, b);
}

hipError_t launch_attn16(const BatchArgs& b, int32_t head_dim, bool fp16, bool transient,
                         hipStream_t stream) {
  if (head_dim != 64) return hipErrorInvalidValue;
  const dim3 grid(8 * b.items_per_xcd), block(kThreads16);
  // the single loading wavefront when every stream's largest query group
  // holds at most 11 halves (the kernel deals them as ceil(halves / groups));
  // not on skip-append steps, whose instance would then spill registers
  bool one = !transient;
  for (int32_t i = 0; i < b.n; ++i) {
    const int32_t n_half = (b.s[i].Tq + 31) / 32;
    one = one && (n_half + b.s[i].n_qt - 1) / b.s[i].n_qt <= 11;
  }
  if (fp16 && transient)
    hipLaunchKernelGGL((attn_d64_kernel<_Float16, true, false>), grid, block, 0, stream, b);
  else if (fp16)
    launch_inst<_Float16>(b, one, grid, block, stream);
  else if (transient)
    hipLaunchKernelGGL((attn_d64_kernel<__bf16, true, false>), grid, block, 0, stream, b);
  else
    launch_inst<__bf16>(b, one, grid, block, stream);
  return hipGetLastError();
}

int32_t attn_occupancy16() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_d64_kernel<__bf16, false, false>, kThreads16, 0) !=
          hipSuccess ||
      n < 1)
    return 1;
  return n;
}

}  // namespace lbm
