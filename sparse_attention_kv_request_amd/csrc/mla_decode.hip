// Sparse MLA decode attention over the rows a swap call returned.
//
// "SGLang HiSparse" blog, section 1 (attention is exact over the positions
// the indexer selected) and section 2.1 (the sparse table a swap-in returns
// goes straight to decode attention).  Absorbed-MLA decode form: each KV row
// holds a 512-dim latent c and a 64-dim rope key r; for head h
//   s_i = scale * (q_h[:512].c_i + q_h[512:].r_i),  out_h = softmax(s) . c,
//   lse_h = log sum exp(s).
//
// Work split: one workgroup = 4 waves (one per SIMD) = 128 heads of one batch
// row over one range of its locations (split-K over locations when the batch
// is small; a second kernel merges the splits by their log-sum-exp).  The
// rows of the range are resolved once.  Tiles of 32 rows are gathered from
// the hot buffer straight into LDS with 16-byte global->LDS loads (no VGPR
// staging), double buffered so the next tile streams in while the current
// one is computed; fp8 rows land two tiles ahead in raw buffers, and every
// thread dequantises the next tile to bf16 between the current tile's P.V
// MFMAs.  Each wave owns 32 heads and computes with MFMA
// 32x32x16 bf16 (one wave per SIMD issues it at 82-86 % of the matrix peak,
// MFMA 16x16x32 at 54 %):
//   S^T (32 tokens x 32 heads) = K (tokens x 576) . Q^T  -- Q^T held in VGPRs
//   O^T (dims x heads)        += V^T (dims x tokens) . P^T -- O^T in AGPRs
// V^T operands come from the same token-major tile through the transposing
// LDS read: a 16-lane group that reads a 4-token x 16-dim block hands every
// lane the 4 tokens of one dim.  With heads as the N dimension every lane's
// accumulators belong to one head (lane l: head l%32), so the softmax
// reductions are in-lane plus one exchange with lane l ^ 32, and the C layout
// of S^T is directly the B operand of the P.V product (the P.V contraction
// takes the tokens in the order the lanes hold them).
#include <type_traits>

#include "internal.h"

// Opt-in instrumentation, a separate build (-DHISPARSE_PHASE_CLOCKS=1, see
// phase_clocks.py): in the bf16 tile loop every wave of the last launch
// stores the shader clocks it spent waiting for a tile's gather, at the
// phase barriers and in the whole loop (hisparse_attention_wait_clocks()),
// and every workgroup the 100 MHz wall clock at its start (stamp 0), at the
// first tile's barrier (1), after the tile loop (2), at its end (3), and in
// the setup once its rows are computed from the locations (6), after the row
// table's barrier (4) and once the queries and the first tile have landed
// in its first wave (5, bf16 rows) (hisparse_attention_phase_clocks()).  The
// default build records nothing.
#ifndef HISPARSE_PHASE_CLOCKS
#define HISPARSE_PHASE_CLOCKS 0
#endif
#if HISPARSE_PHASE_CLOCKS
constexpr int kAttnClockRows = 4096;
__device__ unsigned long long g_attn_wave[kAttnClockRows * 4 * 3];
extern "C" int hisparse_attention_wait_clocks(unsigned long long* out_h, int n) {
  if (n < 0 || n > kAttnClockRows * 4 * 3) return -1;
  return hipMemcpyFromSymbol(out_h, HIP_SYMBOL(g_attn_wave), n * sizeof(unsigned long long)) ==
                 hipSuccess
             ? 0 : -1;
}
constexpr int kAttnStamps = 7;
__device__ long long g_attn_stamp[kAttnClockRows * kAttnStamps];
#define ATTN_CLOCK(i)                                                            \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kAttnClockRows)                        \
      g_attn_stamp[blockIdx.x * kAttnStamps + (i)] = wall_clock64();            \
  } while (0)
extern "C" int hisparse_attention_phase_clocks(long long* out_h, int n) {
  if (n < 0 || n > kAttnClockRows * kAttnStamps) return -1;
  return hipMemcpyFromSymbol(out_h, HIP_SYMBOL(g_attn_stamp), n * sizeof(long long)) == hipSuccess
             ? 0 : -1;
}
#else
#define ATTN_CLOCK(i) \
  do {                \
  } while (0)
#endif

namespace hisparse {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;     // 576
constexpr int kTile = 32;                 // rows per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;  // 256
constexpr int kHeadsPerWave = 32;
constexpr int kHeadsPerGroup = kHeadsPerWave * kWaves;
constexpr int kKSteps = kDim / 16;        // 36 k-steps of MFMA 32x32x16
constexpr int kDimBlocks = kLatent / 32;  // 16 blocks of 32 output dims
constexpr int kMaxPerSplit = 2048;        // locations one workgroup handles
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kQkAhead = 2;               // k-steps of K operands read ahead
constexpr int kPvAhead = 4;               // dim blocks of V operands read ahead
constexpr int kSchedMfma = 0x008;         // scheduling-group masks: MFMA
constexpr int kSchedDsRead = 0x100;       // LDS read
constexpr float kRefSlack = 64.f;         // log2 headroom of the weights over their reference

// bf16 tile: row pitch 608 elements = 1216 B = 76 16-byte slots, and the
// 16-byte chunk c of row r sits in slot c ^ ((r >> 2) & 3) of its row.  With
// 64 banks of 4 bytes a slot covers one of 16 four-bank groups, slot p of row
// r group (12 r + p) mod 16.  That makes both operand reads conflict-free:
// the K reads (16 lanes: 16 consecutive rows, one chunk) hit 16 groups since
// 12 r takes every multiple of 4 once per 4 rows and the XOR separates the
// four rows that share one; the transposing V reads (32 lanes: 4 consecutive
// rows x 4 aligned chunks) keep each row's chunks inside one aligned 4-group
// and put the 4 rows 12 apart.  (A 73-slot pitch without the XOR gave the V
// reads a two-way conflict.)  A global->LDS load instruction fills 64
// consecutive slots, so a tile takes 38 of them; the swizzle lives in the
// global offsets each lane loads.
constexpr int kPitch = kDim + 32;
constexpr int kRowSlots = kPitch / 8;                                  // 76
constexpr int kTileInstr = (kTile * kRowSlots + kWave - 1) / kWave;    // 38
constexpr int kTileBytes = kTileInstr * kWave * 16;                    // 38912

// Slot of 16-byte chunk c of tile row r (c < 72; aligned 4-chunk groups map
// to themselves).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }
// raw fp8 tile: rows of 656 B = 41 slots back to back
constexpr int kFp8Row = kLatent + 16 + 2 * kRope;                      // 656
constexpr int kFp8Slots = kFp8Row / 16;                                // 41
constexpr int kRawInstr = (kTile * kFp8Slots + kWave - 1) / kWave;     // 21
constexpr int kRawBytes = kRawInstr * kWave * 16;                      // 21504
// LDS: bf16 rows use two tile buffers; fp8 rows two tiles + two raw buffers
template <bool fp8>
constexpr int kStageBytes = fp8 ? 2 * kTileBytes + 2 * kRawBytes : 2 * kTileBytes;

struct MlaArgs {
  const uint16_t* q;          // bf16 bits [B][Hq][576]
  const int32_t* locs;        // [B][n_locs]
  const int32_t* page_table;  // [B][pt_stride] or null (token rows)
  const uint8_t* kv;          // the layer's hot buffer
  int64_t kv_rows;            // token rows in kv
  int32_t item_bytes;         // 1152 (bf16) or 656 (fp8)
  int32_t page_size;
  int32_t pt_stride;
  int32_t batch, heads, n_locs, splits, per_split, groups, units;
  float scale_log2;           // softmax scale * log2(e)
  float* out;                 // [B][Hq][512]
  float* lse;                 // [B][Hq] or null
  _Float16* part_out;         // [B][splits][Hq][512] normalised split outputs (fp16)
  float* part_ml;             // [B][splits][Hq][8]: running max (log2 units), sum, 0,
                              // 0, then 16 int8 exponents e: 32-dim block db of the
                              // fp16 output is stored scaled by 2^-e[db]
  uint32_t* err;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats rounded to bf16 (nearest even), low one in the low half: one
// pair conversion (v_cvt_pk_bf16_f32) rather than two conversions, a shift
// and an OR.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Token rows of this thread's locations (-1: skipped or out of range).
// Token rows are the locations themselves; in page mode every page-table
// load goes out before the first is used (a buffer load per location with
// no per-lane branch: a location whose page index lies outside the row's
// table reads past the buffer, which returns zero, and is masked), so the
// lookups cost one round trip rather than one each.
template <int kN>
__device__ __forceinline__ void token_rows(const MlaArgs& a, int b, const int32_t (&loc)[kN],
                                           int64_t (&row)[kN]) {
  if (a.page_table == nullptr) {
#pragma unroll
    for (int k = 0; k < kN; ++k) row[k] = loc[k] >= 0 && loc[k] < a.kv_rows ? loc[k] : -1;
    return;
  }
  const __amdgpu_buffer_rsrc_t pt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.page_table + static_cast<size_t>(b) * a.pt_stride), 0,
      4 * a.pt_stride, 0x00020000);
  int32_t page[kN];
#pragma unroll
  for (int k = 0; k < kN; ++k) {
    const int j = loc[k] >= 0 ? loc[k] / a.page_size : a.pt_stride;
    page[k] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(
        pt, 4 * (j < a.pt_stride ? j : a.pt_stride), 0, 0));
  }
#pragma unroll
  for (int k = 0; k < kN; ++k) {
    const int j = loc[k] >= 0 ? loc[k] / a.page_size : a.pt_stride;
    const int64_t r = static_cast<int64_t>(page[k]) * a.page_size + (loc[k] - j * a.page_size);
    row[k] = j < a.pt_stride && page[k] >= 0 && r < a.kv_rows ? r : -1;
  }
}

// This wave's share of the loads of tile rows [t0, t0 + 32) straight into
// LDS (buffer loads with the LDS bit, 16 bytes per lane): instruction i
// fills slots 64i .. 64i + 63 of the buffer, lane l slot 64i + l.  `rowoff`
// holds each location's byte offset in the hot buffer, or kAbsent (padding,
// skipped locations, and the table's tail past the last location); the
// bf16 pitch pad adds kAbsent too.  Offsets of 2^31 and above fail the
// buffer range check and read zeros, so absent rows meet their zero weights
// with zero values.  (A pad slot of an absent row wraps to a small offset
// and loads harmless bytes that nothing reads.)  All loads of the next tile
// are issued right after the phase barrier: interleaved with the QK LDS
// reads they would make the compiler wait for them before each read.
constexpr uint32_t kAbsent = 0x80000000u;  // beyond every hot buffer (< 2 GiB)

template <int kSlots, int kInstr>
struct TileLoader {
  static constexpr int kRowBytes = kSlots == kFp8Slots ? kFp8Row : 2 * kDim;
  static constexpr int kPerWave = (kInstr + kWaves - 1) / kWaves;
  uint32_t off[kPerWave];
  uint8_t* buf;

  // Offsets of this wave's loads of tile rows [t0, t0 + 32) into `dst`
  // (rowoff reads only); returns the tile's valid-row mask.
  __device__ __forceinline__ uint32_t prepare(const uint32_t* rowoff, int t0, uint8_t* dst,
                                              int wave, int lane) {
    buf = dst;
#pragma unroll
    for (int k = 0; k < kPerWave; ++k) {
      const int s = kWave * (wave + kWaves * k) + lane;
      const int r = s / kSlots;
      const int c = s - r * kSlots;
      // bf16 rows: slot c holds chunk swz(r, c) (an involution; pad slots
      // 72..75 stay past the row)
      const int lc = kSlots == kFp8Slots ? c : swz(r, c);
      off[k] = rowoff[t0 + r] + (16 * lc < kRowBytes ? 16u * lc : kAbsent);
    }
    const bool present = lane < kTile && rowoff[t0 + (lane & (kTile - 1))] != kAbsent;
    return static_cast<uint32_t>(__ballot(present));
  }
  // Load k of this wave.  Issued as inline assembly so that the compiler
  // does not track these LDS writes: it cannot tell the two tile buffers
  // apart and would make the transposing LDS reads of the current tile wait
  // for the next tile's gather.  Completion is awaited explicitly (vmcnt 0)
  // before the barrier that publishes a tile.
  __device__ __forceinline__ void fire(__amdgpu_buffer_rsrc_t kv, int k, int wave) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (LDS_AS uint8_t*)(buf + (wave + kWaves * k) * kWave * 16))));
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off[k]), "s"(kv), "{m0}"(lds)
                 : "memory");
  }
  // The loads from k0 on that this wave has.
  __device__ __forceinline__ void fire_rest(__amdgpu_buffer_rsrc_t kv, int k0, int wave) {
#pragma unroll
    for (int k = 0; k < kPerWave; ++k)
      if (k >= k0 && wave + kWaves * k < kInstr) fire(kv, k, wave);
  }
};

// fp8 rows: the raw tile (codes, 4 scales, bf16 rope per row) -> bf16 tile,
// as 9 jobs per thread.  Job k < 8 of thread t: latent chunk j = t + 256 k
// (8 codes of row j / 64, chunk j % 64; consecutive lanes take consecutive
// chunks of a row); job 8: rope chunk t % 8 of row t / 8 (16 bytes).
constexpr int kDequantJobs = kTile * (kLatent / 8) / kThreads + 1;  // 9
constexpr int kJobStride = 2;  // P.V operands per dequantisation job
static_assert(kDequantJobs * kJobStride <= 2 * kDimBlocks, "jobs must fit the P.V loop");
__device__ __forceinline__ void dequant_job(const uint8_t* raw, uint16_t* tile, int k) {
  const int tid = threadIdx.x;
  if (k < kDequantJobs - 1) {
    const int j = tid + kThreads * k;
    const int r = j >> 6, c = j & 63;
    const uint8_t* src = raw + r * kFp8Row;
    const u32x2 codes = *reinterpret_cast<const u32x2*>(src + 8 * c);
    const float sc = *reinterpret_cast<const float*>(src + kLatent + 4 * (c >> 4));
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f32x2 x0 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);
      const f32x2 x1 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);
      o[2 * w] = pack_bf16(x0[0] * sc, x0[1] * sc);
      o[2 * w + 1] = pack_bf16(x1[0] * sc, x1[1] * sc);
    }
    *reinterpret_cast<u32x4*>(tile + r * kPitch + 8 * swz(r, c)) = o;
  } else {
    const int r = tid >> 3, c = tid & 7;
    *reinterpret_cast<u32x4*>(tile + r * kPitch + 8 * swz(r, kLatent / 8 + c)) =
        *reinterpret_cast<const u32x4*>(raw + r * kFp8Row + kLatent + 16 + 16 * c);
  }
}

// Value of lane l ^ 32 / l ^ 16 (gfx950 row swaps: with both operands x,
// permlane32_swap returns (x of lanes 0-31 twice, x of lanes 32-63 twice),
// so lane l holds x[l] in one result and x[l ^ 32] in the other; permlane16
// does the same for the 16-lane rows 0/1 and 2/3).
__device__ __forceinline__ float xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

// K operand (A of MFMA 32x32x16) of k-step ks: tile row lane%32, chunk 2 ks +
// lane/32, whose slot is 4 (ks/2) + ((2 (ks%2) + lane/32) ^ swizzle): kb[p]
// points at the slot of chunk 2 p + lane/32 of that row.
__device__ __forceinline__ bf16x8 k_operand(const uint16_t* const kb[2], int ks) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(kb[ks & 1] + 32 * (ks >> 1)));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// V^T operand (A of MFMA 32x32x16) of a 32-dim block and 16 tokens: two
// transposing reads, at plo and at phi (8 rows below, with that row's
// swizzle), giving k-slots 0..3 and 4..7.
__device__ __forceinline__ bf16x8 v_operand(const uint16_t* plo, const uint16_t* phi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(plo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(phi));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

template <bool fp8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode(MlaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kStageBytes<fp8>];
  __shared__ uint32_t rowoff[kMaxPerSplit + 2 * kTile + 1];  // byte offset of each location's row
  __shared__ int32_t restart_at[2];

  // XCD-aware mapping (workgroups are dealt to the 8 XCDs round robin):
  // every split and head group of batch row b runs on XCD b mod 8, so the
  // row's queries are fetched from HBM once and shared through that XCD's
  // L2.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int kx = id >> 3;
  const int hg = kx % a.groups;
  const int su = kx / a.groups;
  const int split = su % a.splits;
  const int b = (su / a.splits) * 8 + xcd;
  if (b >= a.batch) return;
  ATTN_CLOCK(0);
  const int t_begin = split * a.per_split;
  const int nrows = max(0, min(a.n_locs, t_begin + a.per_split) - t_begin);
  const int tid = threadIdx.x;
  if (tid < 2) restart_at[tid] = -2;

  // byte offsets of this split's rows (kAbsent = skipped), padded with
  // kAbsent up to two tiles past the last one (plus the one row a raw fp8
  // gather's last instruction reaches into).  Every location load goes out
  // before the first is used (one round trip, not one per pass), and so do
  // the page-table loads of page mode.
  constexpr int kRowIters = (kMaxPerSplit + 2 * kTile + 1 + kThreads - 1) / kThreads;
  const int padded = (nrows + kTile - 1) / kTile * kTile + 2 * kTile + 1;
  const int32_t* lrow = a.locs + static_cast<size_t>(b) * a.n_locs + t_begin;
  int32_t locv[kRowIters];
#pragma unroll
  for (int k = 0; k < kRowIters; ++k) {
    const int t = tid + k * kThreads;
    locv[k] = t < nrows ? lrow[t] : -1;
  }

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar branches
  const int hl = lane & 31;      // head of the wave's 32 / tile row of the K operand
  const int h2 = lane >> 5;      // k-slot half

  // Q^T operands (B of S^T = K . Q^T): lane holds q[head][16 ks + 8 (lane/32)
  // .. +8] of head lane%32 of the wave's 32 (issued behind the location
  // loads, so the row table waits for the locations only and the queries
  // land behind the first tile's gather; nothing uses them before the first
  // tile).  A lane past the last head loads head 0: its results are never
  // stored, and its scores equal head 0's, so it cannot ask for a restart
  // head 0 would not ask for.
  bf16x8 qreg[kKSteps];
  {
    const int head = hg * kHeadsPerGroup + wave * kHeadsPerWave + hl;
    const uint16_t* qh =
        a.q + (static_cast<size_t>(b) * a.heads + (head < a.heads ? head : 0)) * kDim + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 16 * ks));
  }

  int64_t rowv[kRowIters];
  token_rows(a, b, locv, rowv);
  ATTN_CLOCK(6);
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kRowIters; ++k) {
    const int t = tid + k * kThreads;
    bad |= rowv[k] < 0 && locv[k] >= 0;
    if (t < padded)
      rowoff[t] = rowv[k] >= 0
                      ? static_cast<uint32_t>(rowv[k]) * static_cast<uint32_t>(a.item_bytes)
                      : kAbsent;
  }
  if (bad) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);

  __syncthreads();  // rows[] complete
  ATTN_CLOCK(4);

  // O^T of the wave's 32 heads: block db holds dims 32 db + [0, 32); its
  // register j at lane l is dim 32 db + 8 (j/4) + 4 (l/32) + j%4 of head l%32
  f32x16 acc[kDimBlocks];
#pragma unroll
  for (int i = 0; i < kDimBlocks; ++i) acc[i] = zero16();
  float m_ref = -INFINITY;  // reference of the weights of head lane%32, log2 units
  float l_run = 0.f;        // sum of its weights (fp32, before the bf16 rounding)

  const __amdgpu_buffer_rsrc_t kv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.kv), 0, static_cast<int>(a.kv_rows * a.item_bytes), 0x00020000);
  using Loader = std::conditional_t<fp8, TileLoader<kFp8Slots, kRawInstr>,
                                    TileLoader<kRowSlots, kTileInstr>>;
  Loader ld;
  const int ntiles = (nrows + kTile - 1) / kTile;
  // The weights are exp2(s - m_ref) with m_ref fixed per head at the first
  // tile's maximum, so the accumulators are never rescaled (they sit in
  // AGPRs, where a read-modify-write would cost more than the whole tile).
  // Weights may exceed 1 by up to 2^kRefSlack; a tile whose maximum goes
  // beyond that asks for a restart: it raises the wave's reference and
  // posts the phase in restart_at[phase & 1].  Every wave reads the request
  // after a later barrier and replays the range from the start with zeroed
  // sums and accumulators (a write-only reset; a replay that a later phase
  // requests again is harmless: it restarts the sums once more).
  //
  // One tile (bf16, in LDS): S^T, softmax and O^T += V^T P^T; job(o) runs
  // beside the P.V MFMA of operand o.
  // bf16: operand reads and MFMAs pinned in turn; fp8: left to the
  // scheduler between the fenced dequantisation jobs
  constexpr bool kPinPv = !fp8;
  auto tile_step = [&](const uint16_t* tile, uint32_t valid, bool fresh, int phase,
                       auto&& job) {
    // S^T (32 tokens x the wave's 32 heads) = K . Q^T: 36 k-steps of MFMA
    // 32x32x16 in one accumulation chain, K operands read
    // kQkAhead steps ahead (one wave per SIMD: nothing else hides the LDS
    // latency), the interleave pinned by scheduling-group barriers.
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s0 = zero16();
    {
      const int ksw = (hl >> 2) & 3;
      const uint16_t* const kbase[2] = {tile + hl * kPitch + 8 * (h2 ^ ksw),
                                        tile + hl * kPitch + 8 * ((2 + h2) ^ ksw)};
      bf16x8 kf[kQkAhead + 1];
#pragma unroll
      for (int j = 0; j < kQkAhead; ++j) kf[j] = k_operand(kbase, j);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kQkAhead < kKSteps) kf[(ks + kQkAhead) % (kQkAhead + 1)] = k_operand(kbase, ks + kQkAhead);
        s0 = mfma32(kf[ks % (kQkAhead + 1)], qreg[ks], s0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kQkAhead, 0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kQkAhead < kKSteps) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Weights of head lane%32: register j holds token 8 (j/4) + 4 (lane/32) +
    // j%4, lane ^ 32 the other 16 tokens.  The maximum is taken over the
    // unscaled scores (the scale is positive) and the scale folds into one
    // FMA in front of the exponential; a tile whose rows are all present
    // skips the per-score masking.
    const bool full = valid == 0xFFFFFFFFu;
    float raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = s0[j];
    if (!full) {
      const uint32_t lv = valid >> (4 * h2);  // bit 8 (j/4) + j%4: register j's row
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (!((lv >> (8 * (j >> 2) + (j & 3))) & 1u)) raw[j] = -INFINITY;
    }
    float m8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m8[j] = fmaxf(raw[j], raw[j + 8]);
    float rmax = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])),
                       fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    rmax = fmaxf(rmax, xor32(rmax));
    const float tmax = rmax * a.scale_log2;
    const bool beyond = tmax > m_ref + kRefSlack;
    const bool restart = beyond && m_ref != -INFINITY;
    if (beyond) m_ref = tmax;
    // no reference yet means no valid row yet: every score is -inf, every p 0
    const float mr = m_ref == -INFINITY ? 0.f : m_ref;
    float psum = 0.f;
    u32x4 pbits[2];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      // v_exp_f32: results below the smallest normal flush to 0
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(raw[j], a.scale_log2, -mr));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(raw[j + 1], a.scale_log2, -mr));
      const uint32_t pw = pack_bf16(p0, p1);
      pbits[j >> 3][(j & 7) >> 1] = pw;
      // The normaliser sums the fp32 weights (before their bf16 rounding),
      // each written as its rounded value plus the remainder: p - bf16(p) is
      // exact in fp32 and so is the sum, i.e. the same value as p, but the
      // scheduler then keeps the packed word instead of both fp32 weights
      // live over the loop (the fp8 kernel spills registers otherwise).
      const float b0 = __builtin_bit_cast(float, pw << 16);
      const float b1 = __builtin_bit_cast(float, pw & 0xFFFF0000u);
      psum += b0 + (p0 - b0);
      psum += b1 + (p1 - b1);
    }
    psum += xor32(psum);
    l_run = fresh ? psum : l_run + psum;
    const bf16x8 pop[2] = {__builtin_bit_cast(bf16x8, pbits[0]), __builtin_bit_cast(bf16x8, pbits[1])};
    if (__any(restart) && lane == 0) restart_at[phase & 1] = phase;

    // O^T += V^T . P^T, MFMA 32x32x16: for token half u, k-slot 8 (lane/32)
    // + i is token 16u + 4 (lane/32) + i (i < 4) or 16u + 8 + 4 (lane/32) +
    // i - 4, the tokens of the lane's S^T registers 8u .. 8u + 7, so P^T
    // comes straight from the softmax.  The V^T operand of (block db, half
    // u) is two transposing reads: lane j of 16-lane group q points at row
    // 16u + 4 (q/2) + j/4 (then 8 rows below), dims 32 db + 16 (q%2) +
    // 4 (j%4) .. +3, and receives dim 32 db + lane%32 of those 4 rows.
    // Those dims are half j%2 of chunk 4 db + 2 (q%2) + (j%4)/2, whose slot
    // differs from it only in the low two bits (the row's swizzle, (q/2) for
    // the first read and (q/2 + 2) mod 4 for the second, whatever u and db).
    // Operands run half-major, so consecutive MFMAs feed different blocks.
    const int q16 = lane >> 4, j16 = lane & 15;
    const int vc = 2 * (q16 & 1) + ((j16 & 3) >> 1);
    const uint16_t* vlo = tile + (4 * (q16 >> 1) + (j16 >> 2)) * kPitch +
                          8 * (vc ^ ((q16 >> 1) & 3)) + 4 * (j16 & 1);
    const uint16_t* vhi = tile + (4 * (q16 >> 1) + (j16 >> 2) + 8) * kPitch +
                          8 * (vc ^ (((q16 >> 1) + 2) & 3)) + 4 * (j16 & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (fresh) {  // replay: the sums start over
#pragma unroll
      for (int db = 0; db < kDimBlocks; ++db) acc[db] = zero16();
    }
    {
      constexpr int kOps = 2 * kDimBlocks;  // operand o: half o / 16, block o % 16
      auto vop = [&](int o) {
        const int d = 16 * (o / kDimBlocks) * kPitch + 32 * (o % kDimBlocks);
        return v_operand(vlo + d, vhi + d);
      };
      bf16x8 vf[kPvAhead + 1];
#pragma unroll
      for (int j = 0; j < kPvAhead; ++j) vf[j] = vop(j);
#pragma unroll
      for (int o = 0; o < kOps; ++o) {
        if (o + kPvAhead < kOps) vf[(o + kPvAhead) % (kPvAhead + 1)] = vop(o + kPvAhead);
        acc[o % kDimBlocks] =
            mfma32(vf[o % (kPvAhead + 1)], pop[o / kDimBlocks], acc[o % kDimBlocks]);
        job(o);
      }
      if constexpr (kPinPv) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPvAhead, 0);
#pragma unroll
      for (int o = 0; o < kOps; ++o) {
        if (o + kPvAhead < kOps) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (!fp8) {
    // bf16 rows are gathered straight into the two tile buffers (stage + {0,
    // kTileBytes}), one tile ahead.  A restart request read after a phase's
    // barrier fetches the first tile again instead of the next one and, one
    // phase later, replays from it; a request posted by the last tile is
    // read after one more barrier at the end of the range.
    auto dst = [&](int buf) { return stage + buf * kTileBytes; };
    uint32_t valid_next = 0u;  // valid rows of the tile in flight
    if (ntiles > 0) {
      valid_next = ld.prepare(rowoff, 0, dst(0), wave, lane);
      ld.fire_rest(kv, 0, wave);
    }
    // The query loads and the first tile are awaited by the compiler's own
    // wait instruction here, so that it knows the query registers are loaded
    // and puts no waits for them inside the loop (where they would also wait
    // for the gather).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    ATTN_CLOCK(5);
    int it = 0;          // tile in buffer `cur`
    bool fresh = false;  // this phase starts the sums over
#if HISPARSE_PHASE_CLOCKS
    unsigned long long c_gather = 0, c_barrier = 0;
    const unsigned long long c_loop = __builtin_amdgcn_s_memtime();
#endif
    for (int phase = 0; it < ntiles; ++phase) {
      const int cur = phase & 1;
#if HISPARSE_PHASE_CLOCKS
      const unsigned long long c0 = __builtin_amdgcn_s_memtime();
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const unsigned long long c1 = __builtin_amdgcn_s_memtime();
      __syncthreads();
      c_gather += c1 - c0;
      c_barrier += __builtin_amdgcn_s_memtime() - c1;
      if (phase == 0) ATTN_CLOCK(1);
#else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // this phase's tile is in LDS; every wave is done with the last one
#endif
      const bool replay = restart_at[cur ^ 1] == phase - 1;
      const int next = replay ? 0 : it + 1;
      const uint32_t valid = valid_next;  // bit t: row t of this tile is present
      // loads of the next tile (past the last tile: all absent, harmless
      // zeros into the idle buffer)
      valid_next = ld.prepare(rowoff, next * kTile, dst(cur ^ 1), wave, lane);
      ld.fire_rest(kv, 0, wave);
      tile_step(reinterpret_cast<const uint16_t*>(dst(cur)), valid, fresh, phase, [](int) {});
      fresh = replay;
      it = next;
      if (it >= ntiles) {
        // end of the range: the gather of the all-absent tile past it lands,
        // and a request posted by the last tile sends the range round again
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (restart_at[cur] == phase) {
          valid_next = ld.prepare(rowoff, 0, dst(cur ^ 1), wave, lane);
          ld.fire_rest(kv, 0, wave);
          it = 0;
          fresh = true;
        }
      }
    }
#if HISPARSE_PHASE_CLOCKS
    ATTN_CLOCK(2);
    if (lane == 0 && blockIdx.x < kAttnClockRows) {
      unsigned long long* wv = g_attn_wave + (blockIdx.x * 4 + wave) * 3;
      wv[0] = c_gather;
      wv[1] = c_barrier;
      wv[2] = __builtin_amdgcn_s_memtime() - c_loop;
    }
#endif
  } else {
    // fp8 rows: raw tiles are gathered two tiles ahead into R(0..1), and the
    // next tile is dequantised into the idle bf16 tile T(pb ^ 1) by every
    // thread in the gaps of the current tile's P.V MFMAs (9 jobs per
    // thread: 8 latent jobs of 8 codes, one 16-byte rope chunk).  A phase
    // computes tile ci from T(pb), dequantises raw tile di = ci + 1 from
    // R(pb ^ 1) and gathers raw tile gi = ci + 2 into R(pb), which the
    // previous phase's dequantisation read before its closing barrier.
    // A restart request read after that barrier sends the next gather to
    // tile 0: the two phases already in flight compute tiles whose sums are
    // dropped, since every phase that computes tile 0 starts the sums over.
    auto T = [&](int i) { return stage + i * kTileBytes; };
    auto R = [&](int i) { return stage + 2 * kTileBytes + i * kRawBytes; };
    uint32_t valid_c = 0u, valid_d = 0u;  // valid rows of tiles ci and di
    if (ntiles > 0) {
      valid_c = ld.prepare(rowoff, 0, R(0), wave, lane);
      ld.fire_rest(kv, 0, wave);
      valid_d = ld.prepare(rowoff, kTile, R(1), wave, lane);
      ld.fire_rest(kv, 0, wave);
    }
    // the compiler's own wait (see the bf16 path): the queries are loaded
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (ntiles > 0) {
      for (int k = 0; k < kDequantJobs; ++k)
        dequant_job(R(0), reinterpret_cast<uint16_t*>(T(0)), k);
    }
    __syncthreads();  // tile 0 dequantised
    int ci = 0, di = 1, gi = 2, pb = 0;
    int pending = 0;  // discarded phases left before tile 0 comes round again
    // at the top of a phase: T(pb) complete, R(pb ^ 1) landed, T(pb ^ 1) and
    // R(pb) idle
    for (int phase = 0; ci < ntiles || pending > 0; ++phase) {
      const uint32_t valid_g = ld.prepare(rowoff, gi * kTile, R(pb), wave, lane);
      ld.fire_rest(kv, 0, wave);
      const uint8_t* raw = R(pb ^ 1);
      uint16_t* nt = reinterpret_cast<uint16_t*>(T(pb ^ 1));
      // job k runs after P.V operand kJobStride k + 1, fenced: hoisting every
      // job's LDS loads ahead would spill (and loading them a job or two
      // early measured slower)
      tile_step(reinterpret_cast<const uint16_t*>(T(pb)), valid_c, ci == 0, phase, [&](int o) {
        if (o % kJobStride == kJobStride - 1 && o / kJobStride < kDequantJobs) {
          __builtin_amdgcn_sched_barrier(0);
          dequant_job(raw, nt, o / kJobStride);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // raw tile gi landed, tile di dequantised, the request posted
      ci = di;
      di = gi;
      gi = gi + 1;
      pb ^= 1;
      valid_c = valid_d;
      valid_d = valid_g;
      if (pending > 0) --pending;
      if (restart_at[phase & 1] == phase) {
        gi = 0;
        pending = 2;
      }
    }
  }

  const int head = hg * kHeadsPerGroup + wave * kHeadsPerWave + hl;
  if (head >= a.heads) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  // block db, register 4 jj + i  <->  dim 32 db + 8 jj + 4 (lane/32) + i
  if (a.splits == 1) {
    float* dst = a.out + (static_cast<size_t>(b) * a.heads + head) * kLatent + 4 * h2;
    if (a.lse != nullptr && h2 == 0)
      a.lse[static_cast<size_t>(b) * a.heads + head] =
          l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : -INFINITY;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * jj) =
            f32x4{acc[db][4 * jj], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]} * inv;
  } else {
    // A split's output goes out in fp16 (relative 2^-11).  A 32-dim block
    // whose largest |value| exceeds fp16's range is stored scaled by a power
    // of two 2^-e that puts that value in [2^14, 2^15) (e = 0 otherwise), so
    // no latent range overflows it.  The split's max and sum stay fp32 and
    // the block exponents (int8) go beside them; the merge multiplies by 2^e
    // again.  Lanes l and l ^ 32 hold the two halves of each block of one
    // head and exchange their maxima, so both take the same e.
    const size_t ps = (static_cast<size_t>(b) * a.splits + split) * a.heads + head;
    if (h2 == 0) *reinterpret_cast<f32x4*>(a.part_ml + 8 * ps) = f32x4{m_ref, l_run, 0.f, 0.f};
    uint32_t ebits[4] = {0u, 0u, 0u, 0u};  // e of block db in byte db % 4 of word db / 4
    // Lanes l and l ^ 32 hold alternating 4-dim groups of one head: one swap
    // of the group each lacks (the fp16 bits of 4 dims, two dwords) gives
    // lane l dims 32 db + 16 p + 8 (l/32) .. +7, one 16-byte store.
    _Float16* dst8 = a.part_out + ps * kLatent + 8 * h2;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db) {
      // the block's maximum comes from the products the conversion uses (a
      // second read of the accumulators makes the compiler spill registers
      // of the tile loop)
      f32x4 g[4];
      float bm = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        g[q4] = f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                      acc[db][4 * q4 + 3]} * inv;
        bm = fmaxf(bm, fmaxf(fmaxf(fabsf(g[q4][0]), fabsf(g[q4][1])),
                             fmaxf(fabsf(g[q4][2]), fabsf(g[q4][3]))));
      }
      bm = fmaxf(bm, xor32(bm));
      if (bm > 65504.f) {
        // frexp: bm = f * 2^x with f in [0.5, 1), so bm * 2^(15 - x) lies in
        // [2^14, 2^15); scaling by a power of two is exact
        const int e = __builtin_amdgcn_frexp_expf(bm) - 15;
        const float r = __builtin_amdgcn_ldexpf(1.f, -e);
        ebits[db >> 2] |= (static_cast<uint32_t>(e) & 0xFFu) << (8 * (db & 3));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) g[q4] *= r;
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const u32x2 b0 = __builtin_bit_cast(u32x2, __builtin_convertvector(g[2 * pr], f16x4));
        const u32x2 b1 = __builtin_bit_cast(u32x2, __builtin_convertvector(g[2 * pr + 1], f16x4));
        const u32x2 send = h2 == 0 ? b1 : b0;
        u32x2 recv;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto rr = __builtin_amdgcn_permlane32_swap(send[w], send[w], false, false);
          recv[w] = h2 ? rr[0] : rr[1];
        }
        const u32x4 out = h2 == 0 ? u32x4{b0[0], b0[1], recv[0], recv[1]}
                                  : u32x4{recv[0], recv[1], b1[0], b1[1]};
        *reinterpret_cast<u32x4*>(dst8 + 32 * db + 16 * pr) = out;
      }
    }
    if (h2 == 0)
      *reinterpret_cast<u32x4*>(a.part_ml + 8 * ps + 4) =
          u32x4{ebits[0], ebits[1], ebits[2], ebits[3]};
  }
  ATTN_CLOCK(3);
}

// Merges the splits of every (row, head) by their log-sum-exp: 64 lanes per
// head, 8 dims (one 16-byte fp16 load per split) per lane, 4 heads per
// workgroup.  kMaxS > 0 (at most kMaxS splits): every split's record and
// this lane's 16 bytes of it are loaded before any is used, with no branch
// between the loads (split indices past the last repeat it and are then
// skipped), so the merge waits for memory once; kMaxS = 0 loops over any
// number of splits.  Both add the same terms in the same order.
constexpr int kCombineHeads = 4;
template <int kMaxS>
__global__ __launch_bounds__(kCombineHeads * kWave) void mla_combine(MlaArgs a) {
  const int bh = blockIdx.x * kCombineHeads + static_cast<int>(threadIdx.x / kWave);
  if (bh >= a.batch * a.heads) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const size_t ps0 = static_cast<size_t>(b) * a.splits * a.heads + h;  // split s: ps0 + s*heads
  float big = -INFINITY;
  float wsum = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  // split s's term; e: the exponent its 32-dim block is stored scaled by
  auto add = [&](f32x4 ml, int e, u32x4 raw) {
    const float w = exp2f(ml[0] + log2f(ml[1]) - big);
    wsum += w;
    const float wo = __builtin_amdgcn_ldexpf(w, e);
    const f16x4 lo = __builtin_bit_cast(f16x4, u32x2{raw[0], raw[1]});
    const f16x4 hi = __builtin_bit_cast(f16x4, u32x2{raw[2], raw[3]});
    o0 += wo * __builtin_convertvector(lo, f32x4);
    o1 += wo * __builtin_convertvector(hi, f32x4);
  };
  // this lane's 8 dims lie in 32-dim block lane / 4: byte lane / 4 of the
  // record's exponents, i.e. byte (lane / 4) % 4 of exponent word lane / 16
  const int ebyte = 8 * ((lane >> 2) & 3);
  if constexpr (kMaxS > 0) {
    f32x4 ml[kMaxS];
    uint32_t ew[kMaxS];
    u32x4 raw[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      const size_t ps = ps0 + static_cast<size_t>(s < a.splits ? s : a.splits - 1) * a.heads;
      ml[s] = *reinterpret_cast<const f32x4*>(a.part_ml + 8 * ps);  // m, l
      ew[s] = reinterpret_cast<const uint32_t*>(a.part_ml + 8 * ps + 4)[lane >> 4];
      raw[s] = *reinterpret_cast<const u32x4*>(a.part_out + ps * kLatent + 8 * lane);
    }
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      if (s < a.splits && ml[s][1] > 0.f) big = fmaxf(big, ml[s][0] + log2f(ml[s][1]));
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      if (s < a.splits && ml[s][1] > 0.f) add(ml[s], static_cast<int8_t>(ew[s] >> ebyte), raw[s]);
  } else {
    for (int s = 0; s < a.splits; ++s) {
      const size_t ps = ps0 + static_cast<size_t>(s) * a.heads;
      const f32x4 ml = *reinterpret_cast<const f32x4*>(a.part_ml + 8 * ps);
      if (ml[1] > 0.f) big = fmaxf(big, ml[0] + log2f(ml[1]));
    }
    for (int s = 0; s < a.splits; ++s) {
      const size_t ps = ps0 + static_cast<size_t>(s) * a.heads;
      const f32x4 ml = *reinterpret_cast<const f32x4*>(a.part_ml + 8 * ps);
      if (!(ml[1] > 0.f)) continue;
      const uint32_t ew = reinterpret_cast<const uint32_t*>(a.part_ml + 8 * ps + 4)[lane >> 4];
      add(ml, static_cast<int8_t>(ew >> ebyte),
          *reinterpret_cast<const u32x4*>(a.part_out + ps * kLatent + 8 * lane));
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* dst = a.out + static_cast<size_t>(bh) * kLatent + 8 * lane;
  *reinterpret_cast<f32x4*>(dst) = o0 * inv;
  *reinterpret_cast<f32x4*>(dst + 4) = o1 * inv;
  if (a.lse != nullptr && lane == 0) a.lse[bh] = wsum > 0.f ? (big + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

// Splits of the location list per batch row: about one workgroup per CU
// (the kernel runs one workgroup per CU), at least one 32-row tile and at
// most kMaxPerSplit locations per split.
int mla_splits(int batch, int heads, int n_locs, int num_cus) {
  const int groups = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int units = batch * groups;
  int splits = (num_cus + units - 1) / units;
  splits = min(splits, (n_locs + kTile - 1) / kTile);
  splits = max(splits, (n_locs + kMaxPerSplit - 1) / kMaxPerSplit);
  return max(1, splits);
}

int mla_max_locations() { return 64 * kMaxPerSplit; }

size_t mla_workspace_bytes(int batch, int heads, int n_locs, int num_cus) {
  const int splits = mla_splits(batch, heads, n_locs, num_cus);
  if (splits == 1) return 0;
  return static_cast<size_t>(batch) * splits * heads *
         (kLatent * sizeof(_Float16) + 8 * sizeof(float));
}

hipError_t launch_mla_decode(const MlaDecodeCall& c, hipStream_t s) {
  MlaArgs a{};
  a.q = static_cast<const uint16_t*>(c.q);
  a.locs = c.locs;
  a.page_table = c.page_table;
  a.kv = c.kv;
  a.kv_rows = c.kv_rows;
  a.item_bytes = c.item_bytes;
  a.page_size = c.page_size;
  a.pt_stride = c.pt_stride;
  a.batch = c.batch;
  a.heads = c.heads;
  a.n_locs = c.n_locs;
  a.splits = mla_splits(c.batch, c.heads, c.n_locs, c.num_cus);
  a.per_split = ((c.n_locs + a.splits - 1) / a.splits + kTile - 1) / kTile * kTile;
  a.groups = (c.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  a.units = c.batch * a.splits;
  a.scale_log2 = c.scale * 1.44269504088896340736f;
  a.out = c.out;
  a.lse = c.lse;
  a.err = c.err;
  if (a.splits > 1) {
    a.part_out = static_cast<_Float16*>(c.workspace);
    a.part_ml = reinterpret_cast<float*>(a.part_out + static_cast<size_t>(c.batch) * a.splits *
                                                          c.heads * kLatent);
  }
  const int grid = (c.batch + 7) / 8 * 8 * a.splits * a.groups;
  if (c.item_bytes == 2 * kDim)
    hipLaunchKernelGGL(mla_decode<false>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(mla_decode<true>, dim3(grid), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const dim3 cgrid((c.batch * c.heads + kCombineHeads - 1) / kCombineHeads);
  if (a.splits <= 4)
    hipLaunchKernelGGL(mla_combine<4>, cgrid, dim3(kCombineHeads * kWave), 0, s, a);
  else if (a.splits <= 8)
    hipLaunchKernelGGL(mla_combine<8>, cgrid, dim3(kCombineHeads * kWave), 0, s, a);
  else
    hipLaunchKernelGGL(mla_combine<0>, cgrid, dim3(kCombineHeads * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace hisparse
