// Sparse MLA decode attention over the rows a swap call returned.
//
// "SGLang HiSparse" blog, section 1 (attention is exact over the positions
// the indexer selected) and section 2.1 (the sparse table a swap-in returns
// goes straight to decode attention).  Absorbed-MLA decode form: each KV row
// holds a 512-dim latent c and a 64-dim rope key r; for head h
//   s_i = scale * (q_h[:512].c_i + q_h[512:].r_i),  out_h = softmax(s) . c,
//   lse_h = log sum exp(s).
//
// Work split: one workgroup = 8 waves = 128 heads of one batch row over one
// range of its locations (split-K over locations when the batch is small;
// a second kernel merges the splits by their log-sum-exp).  The rows of the
// whole range are resolved once; tiles of 32 rows are gathered into LDS as
// bf16 (fp8 rows dequantised on the way), the next tile's loads in flight in
// registers while the current one is computed.  Each
// wave owns 16 heads and computes with MFMA 16x16x32 bf16:
//   S^T (tokens x heads) = K (tokens x 576) . Q^T   -- the wave's Q^T in registers
//   O^T (dims x heads)  += V^T (dims x tokens) . P^T
// With heads as the N dimension every lane's accumulators belong to one head,
// so the online-softmax rescale is a per-lane scalar, and the C layout of S^T
// is directly the B operand of the P.V product (the 8 tokens a lane holds
// are used as its 8 k-slots, and V^T is read with the same token order).
#include "internal.h"

namespace hisparse {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;     // 576
constexpr int kTile = 32;                 // rows per LDS tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;  // 512
constexpr int kHeadsPerGroup = 16 * kWaves;
constexpr int kRowElems = kDim + 8;       // LDS row pitch in bf16: 292 dwords, so 16
                                          // consecutive rows hit distinct bank groups
constexpr int kKSteps = kDim / 32;        // 18
constexpr int kVtPitch = kTile + 4;       // dim-major latent row: 18 dwords
constexpr int kMaxPerSplit = 2048;        // locations one workgroup handles
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazy = 8.f;              // log2 headroom of the lazy softmax rescale

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
  float* part_out;            // [B][splits][Hq][512]
  float* part_ml;             // [B][splits][Hq][2]: running max (log2 units), sum
  uint32_t* err;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two floats rounded to bf16 (nearest even), low one in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return static_cast<uint32_t>(bf16_bits(lo)) | (static_cast<uint32_t>(bf16_bits(hi)) << 16);
}

// Token row of location `loc` of batch row b, or -1.
__device__ __forceinline__ int64_t token_row(const MlaArgs& a, int b, int32_t loc) {
  if (loc < 0) return -1;
  int64_t row;
  if (a.page_table == nullptr) {
    row = loc;
  } else {
    const int j = loc / a.page_size;
    if (j >= a.pt_stride) return -1;
    const int32_t page = a.page_table[static_cast<size_t>(b) * a.pt_stride + j];
    if (page < 0) return -1;
    row = static_cast<int64_t>(page) * a.page_size + (loc - j * a.page_size);
  }
  return row < a.kv_rows ? row : -1;
}

// Per-thread register staging of one tile's rows: the loads for tile t+1
// are issued before tile t is computed and written to LDS after it.  Thread
// t stages the latent of tokens 2*(t/32) and +1 (bf16 rows: 16-dim chunk t%32
// as two 16-byte words; fp8 rows: 16 codes plus their scale) and, for t < 256,
// rope chunk t%8 of token t/8; it then writes one latent dim of its 2 tokens
// as one 4-byte word of the dim-major copy.
struct Staged {
  u32x4 lat[4];      // bf16: [token x][half c] at 2x+c; fp8: codes of token x at x
  u32x4 rope;
  float scale[2];
};

__device__ __forceinline__ void fetch_tile(const MlaArgs& a, const int32_t* rows, int nrows,
                                           int t0, Staged& st) {
  const int tid = threadIdx.x;
  const int tp = tid >> 5, cp = tid & 31;
  const bool bf16 = a.item_bytes == 2 * kDim;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = t0 + 2 * tp + x;
    const int row = t < nrows ? rows[t] : -1;
    const uint8_t* src = a.kv + static_cast<int64_t>(row) * a.item_bytes;
    if (bf16) {
      st.lat[2 * x] = row >= 0 ? *reinterpret_cast<const u32x4*>(src + 32 * cp) : u32x4{0u, 0u, 0u, 0u};
      st.lat[2 * x + 1] =
          row >= 0 ? *reinterpret_cast<const u32x4*>(src + 32 * cp + 16) : u32x4{0u, 0u, 0u, 0u};
    } else {
      st.lat[x] = row >= 0 ? *reinterpret_cast<const u32x4*>(src + 16 * cp) : u32x4{0u, 0u, 0u, 0u};
      st.scale[x] = row >= 0 ? *reinterpret_cast<const float*>(src + kLatent + (cp >> 3) * 4) : 0.f;
    }
  }
  st.rope = u32x4{0u, 0u, 0u, 0u};
  if (tid < kTile * 8) {
    const int t = t0 + (tid >> 3);
    const int row = t < nrows ? rows[t] : -1;
    const int rope_off = bf16 ? 2 * kLatent : kLatent + 16;
    if (row >= 0)
      st.rope = *reinterpret_cast<const u32x4*>(a.kv + static_cast<int64_t>(row) * a.item_bytes +
                                                rope_off + 16 * (tid & 7));
  }
}

// Column of the 4-token group tg in row d of the dim-major latent copy: the
// group index is XOR-swizzled by (d / 16) mod 8 so that the staging threads'
// stores (rows 16 apart) spread over the banks; readers of one MFMA operand
// all share one d / 16 and stay conflict-free.
__device__ __forceinline__ int vt_col(int d, int tg) { return 4 * (tg ^ ((d >> 4) & 7)); }

// fp8 rows: turn the staged codes of token x (16 latent dims) into packed
// bf16 pairs in place, lat[2x] = dims 0..7, lat[2x+1] = dims 8..15, the
// register format bf16 rows are staged in.
__device__ __forceinline__ void dequant_fp8(Staged& st) {
#pragma unroll
  for (int x = 1; x >= 0; --x) {
    const u32x4 codes = st.lat[x];
    const float sc = st.scale[x];
    u32x4 out[2];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 x0 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);
      const f32x2 x1 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);
      out[w >> 1][2 * (w & 1)] = pack_bf16(x0[0] * sc, x0[1] * sc);
      out[w >> 1][2 * (w & 1) + 1] = pack_bf16(x1[0] * sc, x1[1] * sc);
    }
    st.lat[2 * x] = out[0];
    st.lat[2 * x + 1] = out[1];
  }
}

// Writes the staged tile: token-major rows (all 576 dims) and the dim-major
// latent copy vt[dim][token].  Each 4-byte vt word holds one dim of the
// thread's 2 tokens, assembled with a byte permute of the packed registers.
__device__ __forceinline__ void store_tile(const MlaArgs& a, Staged& st, uint16_t* tile,
                                           uint16_t* vt) {
  const int tid = threadIdx.x;
  const int tp = tid >> 5, cp = tid & 31;
  if (a.item_bytes != 2 * kDim) dequant_fp8(st);
  const int d0 = 16 * cp;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    uint16_t* dst = tile + (2 * tp + x) * kRowElems + d0;
    *reinterpret_cast<u32x4*>(dst) = st.lat[2 * x];
    *reinterpret_cast<u32x4*>(dst + 8) = st.lat[2 * x + 1];
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = e >> 3, w = (e & 7) >> 1;
    // low halves (even dim) or high halves (odd dim) of the two tokens' words
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t v = __builtin_amdgcn_perm(st.lat[2 + c][w], st.lat[c][w], sel);
    const int d = d0 + e;
    *reinterpret_cast<uint32_t*>(vt + d * kVtPitch + vt_col(d, tp >> 1) + 2 * (tp & 1)) = v;
  }
  if (tid < kTile * 8)
    *reinterpret_cast<u32x4*>(tile + (tid >> 3) * kRowElems + kLatent + 8 * (tid & 7)) = st.rope;
}

__global__ __launch_bounds__(kThreads) void mla_decode(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * kRowElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kLatent * kVtPitch];
  __shared__ int32_t rows[kMaxPerSplit];

  // XCD-aware mapping: the head groups of one (row, split) unit run on the
  // same XCD (workgroups are dealt to the 8 XCDs round robin) and share its
  // rows through that XCD's L2.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int k = id >> 3;
  const int hg = k % a.groups;
  const int unit = (k / a.groups) * 8 + xcd;
  if (unit >= a.units) return;
  const int b = unit / a.splits;
  const int split = unit - b * a.splits;
  const int t_begin = split * a.per_split;
  const int nrows = max(0, min(a.n_locs, t_begin + a.per_split) - t_begin);
  const int tid = threadIdx.x;

  // rows of this split's locations (-1 = skipped)
  for (int t = tid; t < nrows; t += kThreads) {
    const int32_t loc = a.locs[static_cast<size_t>(b) * a.n_locs + t_begin + t];
    const int64_t row = token_row(a, b, loc);
    if (row < 0 && loc >= 0) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
    rows[t] = static_cast<int32_t>(row);
  }

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g = lane >> 4;       // lane group
  const int n = lane & 15;       // head within the wave / row within a 16-tile
  const int head = hg * kHeadsPerGroup + wave * 16 + n;
  const bool head_ok = head < a.heads;

  // Q^T operand: lane holds q[head][32*ks + 8*g .. +8] for every k-step
  bf16x8 qreg[kKSteps];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.heads + (head_ok ? head : 0)) * kDim;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qh + 32 * ks + 8 * g);
      if (!head_ok) v = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = as_bf16x8(v);
    }
  }
  __syncthreads();

  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // running sum of the (bf16-rounded) weights

  Staged stage;
  if (nrows > 0) fetch_tile(a, rows, nrows, 0, stage);
  for (int t0 = 0; t0 < nrows; t0 += kTile) {
    store_tile(a, stage, tile, vt);
    __syncthreads();
    if (t0 + kTile < nrows) fetch_tile(a, rows, nrows, t0 + kTile, stage);

    // S^T for tokens [0,16) and [16,32) of the tile
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = tile + (st * 16 + n) * kRowElems + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 kv = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * ks));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qreg[ks], c, 0, 0, 0);
      }
      s[st] = c;
    }
    // online softmax for this lane's head; lane holds tokens 4g+i and 16+4g+i
    float sc[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
      const bool valid = t0 + tok < nrows && rows[t0 + tok] >= 0;
      const float v = valid ? s[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
      sc[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // The weights are taken relative to a reference m_run that only moves
    // when the maximum grows by more than kLazy (log2 units): weights stay
    // below 2^kLazy, and the accumulators are rescaled only on those rare
    // moves (the result is the same; only the common factor differs).
    const bool move = tmax > m_run + kLazy;
    const float m_new = move ? tmax : m_run;
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    float psum = 0.f;
    u16x8 pbits;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = m_new == -INFINITY ? 0.f : exp2f(sc[i] - m_new);
      const uint16_t pb = bf16_bits(p);
      pbits[i] = pb;
      psum += __builtin_bit_cast(float, static_cast<uint32_t>(pb) << 16);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    if (__any(move)) {   // some head of the wave moved its reference
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pbits);

    // O^T += V^T . P^T.  Sub-tile (u, j) covers dims 64u + 16j + [0,16); its
    // A operand row n is dim 64u + 16j + n and its k-slots are the lane's
    // 8 tokens 4g..4g+3 and 16+4g..16+4g+3 (token groups g and 4+g), two
    // 8-byte reads of vt.
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 64 * u + 16 * j + n;
        const uint16_t* vrow = vt + d * kVtPitch;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + vt_col(d, g));
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + vt_col(d, 4 + g));
        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
        acc[4 * u + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), pop,
                                                                 acc[4 * u + j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (head >= a.heads) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* dst;
  if (a.splits == 1) {
    dst = a.out + (static_cast<size_t>(b) * a.heads + head) * kLatent;
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<size_t>(b) * a.heads + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const size_t ps = (static_cast<size_t>(b) * a.splits + split) * a.heads + head;
    dst = a.part_out + ps * kLatent;
    if (g == 0) {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_run;
    }
  }
  // sub-tile (u, j), C row 4g + i  <->  dim 64u + 16j + 4g + i
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4*>(dst + 64 * u + 16 * j + 4 * g) = acc[4 * u + j] * inv;
  }
}

// Merges the splits of every (row, head) by their log-sum-exp.
__global__ __launch_bounds__(128) void mla_combine(MlaArgs a) {
  const int bh = blockIdx.x;  // b * heads + h
  const int b = bh / a.heads, h = bh - b * a.heads;
  float big = -INFINITY;
  for (int s = 0; s < a.splits; ++s) {
    const size_t ps = (static_cast<size_t>(b) * a.splits + s) * a.heads + h;
    const float l = a.part_ml[2 * ps + 1];
    if (l > 0.f) big = fmaxf(big, a.part_ml[2 * ps] + log2f(l));
  }
  float wsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const size_t ps = (static_cast<size_t>(b) * a.splits + s) * a.heads + h;
    const float l = a.part_ml[2 * ps + 1];
    if (!(l > 0.f)) continue;
    const float w = exp2f(a.part_ml[2 * ps] + log2f(l) - big);
    wsum += w;
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.part_out + ps * kLatent + 4 * threadIdx.x);
    o += w * p;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<f32x4*>(a.out + static_cast<size_t>(bh) * kLatent + 4 * threadIdx.x) = o * inv;
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[bh] = wsum > 0.f ? (big + log2f(wsum)) * kLn2 : -INFINITY;
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
  return static_cast<size_t>(batch) * splits * heads * (kLatent + 2) * sizeof(float);
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
    a.part_out = static_cast<float*>(c.workspace);
    a.part_ml = a.part_out + static_cast<size_t>(c.batch) * a.splits * c.heads * kLatent;
  }
  const int padded_units = (a.units + 7) / 8 * 8;
  hipLaunchKernelGGL(mla_decode, dim3(padded_units * a.groups), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine, dim3(c.batch * c.heads), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace hisparse
