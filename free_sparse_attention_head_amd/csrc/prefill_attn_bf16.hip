// sparse_prefill_attn, bf16 inputs: block-sparse causal flash-attention with
// gfx950 direct-to-LDS tile loads and transposing LDS reads.
//
// RBS-Attention post, "Key technical points" 2: the merged block mask is
// executed by an otherwise unchanged block-sparse FlashAttention path.
//
// One workgroup per (batch, query head, query block i): T/32 waves of 32
// query rows.  The workgroup walks the row's causal key blocks in 64-key
// chunks through two LDS buffers:
//   * K and V chunks are copied HBM -> LDS with buffer_load_dwordx4 ... lds
//     (each wave instruction lands 64 lanes x 16 B contiguously): no staging
//     registers, no LDS store instructions, no transposes.  The next chunk's
//     copies are issued before the current chunk is computed;
//   * both tiles are row-major (one key per row) with an XOR swizzle of the
//     16-byte slots, chosen by the source address of each lane, so that the
//     fragment reads below are bank-conflict free;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the wave's Q tile resident
//     as the B operand (each lane then holds one query row's scores);
//   * online softmax in fp32 without a per-chunk row max: the reference
//     exponent is the first chunk's row max, exp2 takes the scale folded into
//     an FMA, and a chunk whose row sum leaves the safe range (a row grew far
//     past the reference, or overflowed) is redone after raising the
//     reference to the true running max and rescaling O^T;
//   * O^T += V^T P^T: P^T comes from registers, V^T fragments come from the
//     row-major V tile through ds_read_b64_tr_b16, which hands lane i of each
//     16-lane group column i of the 4 x 16 tile the group addresses.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fsa {

namespace {

// Largest row-sum share of one chunk in one lane (16 or 32 P values) that is
// accepted against the current reference exponent: P values up to about 2^19
// are exact in fp32 and bf16 alike, and the accumulated sums stay far inside
// the fp32 range.  A larger (or infinite, or NaN) share sends the chunk through
// the reference-raising path.
constexpr float kChunkSumMax = 16777216.0f;  // 2^24
constexpr int kMaxBlocks = 4096;  // key blocks per sequence (S / T) supported
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
#define FSA_LDS __attribute__((address_space(3)))

template <int D, int BLK, int KCH>
struct DirectTraits {
  static constexpr int NW = BLK / 32;         // waves
  static constexpr int NT = NW * 64;          // threads
  static constexpr int KC = KCH;              // keys per chunk (32 or 64)
  static constexpr int NKT = KC / 32;         // 32-key S tiles per chunk
  static constexpr int NCH = BLK / KC;        // chunks per key block
  static constexpr int ROWB = D * 2;          // bytes per key row
  static constexpr int SLOTS = ROWB / 16;     // 16-byte slots per row
  static constexpr int TILE = KC * ROWB;      // bytes of one K (or V) chunk
  static constexpr int RPI = 1024 / ROWB;     // rows per 1 KB load instruction
  static constexpr int IPW = TILE / 1024 / NW;  // load instructions per wave per tile
  static constexpr int BUF = 2 * TILE;        // K + V
  static constexpr size_t LDS = 2 * (size_t)BUF;
  static_assert(IPW >= 1 && TILE % (1024 * NW) == 0, "tile shape");
};

// Slot swizzles.  K rows XOR the slot with the row.  A transposing V read
// touches four consecutive rows (row % 4 = 0..3), 32 or 64 bytes of each per
// 16 or 32 lanes; the V XOR keeps those pieces in distinct banks whether the
// LDS serves 16 lanes from 32 banks or 32 lanes from 64 banks per cycle.
template <int SLOTS>
__device__ __forceinline__ int k_swz(int row) { return row & (SLOTS - 1); }
template <int SLOTS>
__device__ __forceinline__ int v_swz(int row) {
  const int r = row & 3;
  if constexpr (SLOTS == 16) return 4 * r ^ 2 * ((r ^ (r >> 1)) & 1);  // 0, 6, 10, 12
  else return 2 * r;  // 128-byte rows: two rows per 256 bytes already differ
}

// generic -> LDS address-space pointers (a C-style cast is the supported form)
template <typename T>
__device__ __forceinline__ FSA_LDS T* lds_ptr(const void* p) {
  return (FSA_LDS T*)(const_cast<void*>(p));
}

// 16 bytes a lane, HBM -> LDS, through a buffer descriptor (MUBUF form).  A
// non-template function: the host pass then still instantiates the kernels.
__device__ __forceinline__ void copy16_to_lds_buf(__amdgpu_buffer_rsrc_t rs, const void* l, uint32_t voff,
                                                  uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr<void>(l), 16, voff, soff, 0, 0);
}

// 16 bytes a lane, HBM -> LDS (FLAT form): the Q rows of the prologue, which
// are waited for in full before the chunk loop starts.
__device__ __forceinline__ void copy16_to_lds(const void* g, const void* l) {
  __builtin_amdgcn_global_load_lds(g, lds_ptr<void>(l), 16, 0, 0);
}

// max of x over lanes l and l ^ 32: v_permlane32_swap exchanges the two
// halves of the wave in registers (no LDS round trip); of its two results,
// lane l < 32 holds x[l] and x[l + 32], lane l >= 32 holds x[l - 32] and x[l]
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exclusive prefix count of 0/1 flags over the workgroup, for the block-list
// build that runs once per workgroup: a __shfl_up ladder inside each wave and
// one thread walking the wave totals.  Its speed does not matter here; the
// kernel sits at 256 VGPRs, and with the DPP-ladder form of the scan the
// register allocation of the main loop pushed one value to scratch.
__device__ __forceinline__ int list_excl_count(int v, int* tmp, int* total) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6, l = threadIdx.x & 63;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (l >= o) inc += t;
  }
  if (l == 63) tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int x = 0; x < nw; ++x) {
      const int t = tmp[x];
      tmp[x] = run;
      run += t;
    }
    tmp[16] = run;
  }
  __syncthreads();
  const int r = tmp[w] + inc - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

}  // namespace

template <int D, int BLK, int KCH, int LMAX>
__global__ __launch_bounds__(BLK * 2, 2) void prefill_attn_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ bidx,
    const int32_t* __restrict__ bcnt, uint16_t* __restrict__ O, float* __restrict__ LSE, int S,
    int Hq, int Hkv, float scale_log2, int units) {
  using Tr = DirectTraits<D, BLK, KCH>;
  constexpr int KC = Tr::KC, NKT = Tr::NKT, NCH = Tr::NCH, ROWB = Tr::ROWB, SLOTS = Tr::SLOTS;
  constexpr int NP = NKT * 8;  // packed bf16 pairs of P per lane per chunk
  // Two distinct LDS objects for the double buffer: the compiler can then
  // tell that fragment reads of one never alias the copies into the other and
  // keeps the next chunk's copies in flight during the current chunk.
  __shared__ __align__(16) unsigned char kb0[Tr::TILE];
  __shared__ __align__(16) unsigned char kb1[Tr::TILE];
  __shared__ __align__(16) unsigned char vb0[Tr::TILE];
  __shared__ __align__(16) unsigned char vb1[Tr::TILE];
  // the row's key blocks; a static array (not dynamic LDS), so the compiler
  // can also tell list reads apart from the tile copies in flight
  __shared__ uint16_t Ls[LMAX];
  __shared__ int scan_tmp[17];

  // Work order: a unit is one (batch, KV head, query block); units run KV
  // head major, longest query blocks first.  The G query heads of a unit read
  // largely the same K/V blocks, so all G workgroups of a unit go to one XCD
  // (one L2) back to back: workgroups are dealt to the XCDs round-robin, so
  // XCD x takes every kXcds-th unit and its n-th workgroup is head n % G of
  // its (n / G)-th unit.  Every XCD walks the unit order at the same pace.
  const int nB = S / BLK;
  const int G = Hq / Hkv;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int rest = (slot / G) * kXcds + xcd;  // unit
  const int hh = slot % G;
  if (rest >= units) return;
  const int i = nB - 1 - (rest % nB);
  const int bg = rest / nB;
  const int g = bg % Hkv, b = bg / Hkv;
  const int h = g * G + hh;
  const int row = (b * Hq + h) * nB + i;

  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = l & 31, lg = l >> 5;
  const int qrow = wave * 32 + lq;
  const size_t kv_stride = (size_t)Hkv * D;
  const uint16_t* Kb = K + ((size_t)b * S * Hkv + g) * D;
  const uint16_t* Vb = V + ((size_t)b * S * Hkv + g) * D;

  // Each wave owns a 32-row staging region in the K ring (free before the
  // first K/V copies and again after the last S step): its Q rows come in
  // through it and its O rows go out through it, so that every global access
  // of either moves whole token rows (a wave's 32 rows are Hq * D elements
  // apart in HBM; read or written straight from the MFMA layout, each
  // instruction would touch 32 rows at 32 or 16 bytes apart).
  static_assert(Tr::NW <= 2 * NKT, "two K tiles hold every wave's 32 rows");
  constexpr int RPI = Tr::RPI;
  unsigned char* stage = (wave / NKT ? kb1 : kb0) + (wave % NKT) * 32 * ROWB;
  // a wave-uniform base plus a 32-bit per-lane byte offset (row r, 16-byte slot)
  const uint32_t tok_bytes = (uint32_t)(Hq * D) * sizeof(uint16_t);  // token to token
  const size_t row0 = ((size_t)b * S + (size_t)i * BLK + wave * 32) * Hq * D + (size_t)h * D;
  auto row_ofs = [&](int r, int slot) { return (uint32_t)r * tok_bytes + (uint32_t)slot * 16u; };
  // Q rows -> staging region (row-major, the K tile's slot swizzle)
  {
    const char* qsrc = reinterpret_cast<const char*>(Q + row0);
#pragma unroll
    for (int m = 0; m < 32 / RPI; ++m) {
      const int r = m * RPI + l / SLOTS, sl = l % SLOTS;
      copy16_to_lds(qsrc + row_ofs(r, sl ^ k_swz<SLOTS>(r)), stage + m * 1024);
    }
  }

  // the row's causal key blocks, compacted in order into LDS
  const int cnt = bidx ? min(max(bcnt[row], 0), nB) : i + 1;
  int nvalid = 0;
  for (int e0 = 0; e0 < cnt; e0 += Tr::NT) {
    const int e = e0 + tid;
    int j = -1;
    if (e < cnt) j = bidx ? bidx[(size_t)row * nB + e] : e;
    const int ok = (j >= 0 && j <= i) ? 1 : 0;
    FSA_DEBUG_RAISE(e < cnt && !ok, FSA_DBG_BLOCK_INDEX);
    int tot;
    const int pos = list_excl_count(ok, scan_tmp, &tot);
    if (ok) Ls[nvalid + pos] = (uint16_t)j;
    nvalid += tot;
  }
  __syncthreads();
  const int nchunks = nvalid * NCH;

  // staged Q -> registers (MFMA B operand, lane = query row), read like a K
  // fragment; the barrier keeps the ring untouched until every wave has it
  const int kslot_x = lq & (SLOTS - 1);  // K row swizzle of rows lq, lq+32
  // K fragment of MFMA step kk for key row rowp (two 8-element halves: lg)
  auto kfrag = [&](const unsigned char* rowp, int kk) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                          rowp + (((2 * kk + lg) ^ kslot_x) * 16)));
  };
  bf16x8 qf[D / 16];
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) qf[kk] = kfrag(stage + lq * ROWB, kk);
  __syncthreads();

  // HBM -> LDS copy of chunk c into tile buffer kt.  Instruction m of a wave
  // lands rows (wave*IPW + m)*RPI + l/SLOTS of the chunk: the row step of m
  // is a wave-uniform byte offset (the instruction's SGPR offset), and the
  // per-lane part (row l/SLOTS, swizzled slot) is one register for V and one
  // for K, whose slot swizzle changes with m by a constant XOR of the slot
  // bits (a row starts on a multiple of the key stride, itself a multiple
  // of the row size, so the slot bits of the offset are free).
  static_assert((Tr::IPW * Tr::RPI) % SLOTS == 0, "copy rows per wave");
  const uint32_t stride_b = (uint32_t)(kv_stride * sizeof(uint16_t));  // token to token
  uint32_t kofs0, vofs0;
  {
    const int r = wave * Tr::IPW * Tr::RPI + l / SLOTS;
    const int sl = l % SLOTS;
    kofs0 = (uint32_t)r * stride_b + (uint32_t)((sl ^ k_swz<SLOTS>(r)) * 16);
    vofs0 = (uint32_t)r * stride_b + (uint32_t)((sl ^ v_swz<SLOTS>(r)) * 16);
  }
  // The copies are MUBUF loads to LDS through a buffer descriptor of the
  // chunk (base in SGPRs, range = the chunk's rows).  Unlike the FLAT form,
  // the compiler's wait-count model then keeps exact LDS counts for the
  // fragment reads issued while these copies are in flight.
  const uint32_t chunk_bytes = (uint32_t)KC * stride_b;
  // (j = key block of chunk c, read from the list one step ahead)
  auto issue_tile = [&](int c, int j, const uint16_t* src0, bool is_k, unsigned char* tile) {
    j = __builtin_amdgcn_readfirstlane(j);
    const size_t base = ((size_t)j * BLK + (c % NCH) * KC) * stride_b;
    const char* src = reinterpret_cast<const char*>(src0) + base;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, (int)chunk_bytes, 0x00020000);
#pragma unroll
    for (int m = 0; m < Tr::IPW; ++m) {
      // K: the slot swizzle of row r is r % SLOTS, and r moves by m*RPI
      const uint32_t kx = (uint32_t)(((m * Tr::RPI) & (SLOTS - 1)) * 16);
      copy16_to_lds_buf(rs, tile + (wave * Tr::IPW + m) * 1024, is_k ? (kofs0 ^ kx) : vofs0,
                        (uint32_t)(m * Tr::RPI) * stride_b);
    }
  };
  auto issue_k = [&](int c, int j, unsigned char* kt) { issue_tile(c, j, Kb, true, kt); };
  auto issue_v = [&](int c, int j, unsigned char* vt) { issue_tile(c, j, Vb, false, vt); };

  // Pipeline barrier: this wave's tile copies have landed and its LDS reads
  // have retired; the s_barrier then publishes every wave's copies and frees
  // the other buffer.
  auto tile_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  floatx16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  // reference exponent of P in log2 units (scaled score of the reference max),
  // and the row sum of the chunks so far relative to it
  float mref = -INFINITY, l_run = 0.f;
  float l_part = 0.f;  // the current chunk's row-sum share

  // per-lane LDS offsets of the fragment reads
  const int li = l & 15, q16 = (l >> 4) & 1;  // transposing-read lane coordinates
  const int vrow = lg * 4 + (li >> 2);
  const int vcol_b = q16 * 32 + 8 * (li & 3);  // byte column inside a 64-byte dt stripe
  const int vphys_x = v_swz<SLOTS>(li >> 2);   // V row swizzle (row % 4 == li >> 2)
  constexpr int NKK = D / 16;                  // MFMA k-steps of S
  constexpr int NDT = D / 32, NM = (KC / 16) * NDT;  // MFMAs of PV

  // Causal mask (diagonal block only) for chunk c.  Register r of tile tl
  // holds key koff + tl*32 + (r/4)*8 + lg*4 + r%4.  Chunks wholly after this
  // wave's rows come out all masked (P = 0).
  auto causal_mask = [&](int c, int j, floatx16 (&s)[NKT]) {
    const int koff = (c % NCH) * KC;
    if (j == i) {
      const int rel = koff + lg * 4 - qrow;
#pragma unroll
      for (int tl = 0; tl < NKT; ++tl)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rel + tl * 32 + (r >> 2) * 8 + (r & 3) > 0) s[tl][r] = -INFINITY;
    }
  };
  auto row_max = [&](const floatx16 (&s)[NKT]) {
    float mx = -INFINITY;
#pragma unroll
    for (int tl = 0; tl < NKT; ++tl)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tl][r]);
    return max_xor32(mx);
  };
  // The reference exponent is set from the first chunk's row max (before the
  // chunk loop).  Later chunks compute no max (see raise_ref), except the last
  // one (`full`), whose step has no S work to hide a retry behind: it raises
  // the reference to the running max up front.
  auto prelude = [&](int c, int j, floatx16 (&s)[NKT], bool full) -> float {
    causal_mask(c, j, s);
    if (full) {
      const float mx = row_max(s);
      const float m_new = (mx == -INFINITY) ? mref : fmaxf(mref, mx * scale_log2);
      if (__builtin_amdgcn_ballot_w64(m_new > mref) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(mref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        mref = m_new;
      }
    }
    return mref;
  };

  // One sixteenth of the softmax of a chunk: P elements 2q and 2q+1 of the
  // lane's 32 (bf16, packed into pp[q]) and their share of the row sum.  The
  // row sum adds the fp32 values in two partial sums with plain adds:
  // v_dot2 does not issue while an MFMA is in flight, plain VALU does.
  auto p_slice = [&](const floatx16 (&s)[NKT], float mc, uint32_t (&pp)[NP], int q) {
    const int e0 = 2 * q;  // element index kc*8 + e of P
    const float x0 = s[e0 >> 4][e0 & 15], x1 = s[(e0 + 1) >> 4][(e0 + 1) & 15];
    const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, scale_log2, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, scale_log2, -mc));
    bf16x2 pb;
    pb[0] = (__bf16)p0;
    pb[1] = (__bf16)p1;
    pp[q] = __builtin_bit_cast(uint32_t, pb);
    if (q == 0) l_part = p0 + p1;  // the chunk's first slice starts the sum
    else l_part += p0 + p1;
  };

  // A chunk whose row-sum share is out of range: raise the reference to the
  // row's true running max (both wave halves agree on it), rescale O^T and
  // the row sum, and redo the chunk's P.  Returns the chunk's new share.
  auto raise_ref = [&](const floatx16 (&s)[NKT], uint32_t (&pp)[NP]) -> float {
    const float mx = row_max(s);
    const float m_new = (mx == -INFINITY) ? mref : fmaxf(mref, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(mref - m_new);
    mref = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
    for (int q = 0; q < NP; ++q) p_slice(s, mref, pp, q);
    return l_part;
  };

  // S^T = K Q^T of the next chunk from K tile kS into sn (NKT 32x32 tiles:
  // keys 0-31, 32-63), interleaved with the softmax of the current chunk (sc,
  // mc -> pp): after each S MFMA 8 / NKK P slices.  Either half may be
  // absent.  K fragments are read KRD k-steps ahead through a ring; the
  // first KRD steps' fragments are read by the caller, before the prelude.
  constexpr int KRD = 2;
  auto k_first = [&](const unsigned char* kS, bf16x8 (&ring)[KRD][NKT]) {
    const unsigned char* kr0 = kS + lq * ROWB;
#pragma unroll
    for (int kk = 0; kk < KRD; ++kk)
#pragma unroll
      for (int tl = 0; tl < NKT; ++tl) ring[kk][tl] = kfrag(kr0 + tl * 32 * ROWB, kk);
  };
  auto s_and_p = [&](auto has_s, auto has_p, const unsigned char* kS, floatx16 (&sn)[NKT],
                     const floatx16 (&sc)[NKT], float mc, uint32_t (&pp)[NP],
                     bf16x8 (&ring)[KRD][NKT]) {
    constexpr bool DO_S = decltype(has_s)::value, DO_P = decltype(has_p)::value;
    constexpr int SPM = 8 / NKK;  // P slices after each S MFMA (NKT * 8 slices in all)
    static_assert(SPM * NKK == 8, "head dimension");
    const unsigned char* kr0 = kS + lq * ROWB;
    const floatx16 zero = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 a[NKT];
      if constexpr (DO_S) {
#pragma unroll
        for (int tl = 0; tl < NKT; ++tl) a[tl] = ring[kk % KRD][tl];
        if (kk + KRD < NKK) {
#pragma unroll
          for (int tl = 0; tl < NKT; ++tl) ring[kk % KRD][tl] = kfrag(kr0 + tl * 32 * ROWB, kk + KRD);
        }
      }
#pragma unroll
      for (int tl = 0; tl < NKT; ++tl) {
        if constexpr (DO_S)
          sn[tl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tl], qf[kk], kk ? sn[tl] : zero, 0, 0, 0);
        if constexpr (DO_P)
#pragma unroll
          for (int q = 0; q < SPM; ++q) p_slice(sc, mc, pp, (NKT * kk + tl) * SPM + q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O^T += V^T P^T from V tile vt.  PV step m = kc*NDT + dt: the A fragment
  // holds keys kc*16 + lg*4 + {0..3} (first transposing read) and +8
  // (second) at d = dt*32 + lq; fragments are read two MFMAs ahead.
  auto pv = [&](const uint32_t (&pp)[NP], const unsigned char* vt) {
    auto vfrag = [&](int m) {
      const int kc = m / NDT, dt = m % NDT;
      const int r0 = kc * 16 + vrow;
      const int colb = dt * 64 + vcol_b;
      const int slot = (colb >> 4) ^ vphys_x;
      // both addresses as one offset from the tile base, so the compiler can
      // trace them to their LDS buffer
      const int off = r0 * ROWB + slot * 16 + (colb & 15);
      const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_ptr<bf16x4v>(vt + off));
      const bf16x4v hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_ptr<bf16x4v>(vt + (off + 8 * ROWB)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 f0 = vfrag(0), f1 = vfrag(1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bf16x8 f2 = (m + 2 < NM) ? vfrag(m + 2) : f0;
      const int kc = m / NDT;
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, make_uint4(pp[4 * kc], pp[4 * kc + 1], pp[4 * kc + 2], pp[4 * kc + 3]));
      oacc[m % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, pb, oacc[m % NDT], 0, 0, 0);
      f0 = f1;
      f1 = f2;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + 2 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // K and V chunks live in separate two-deep rings (chunk c in kb[c%2] and
  // vb[c%2]).  Step c computes S of chunk c+1 alongside the softmax of chunk
  // c, then PV of chunk c, so at its start K of c+1 and V of c must have
  // landed; it then refills the K slot of chunk c (read by the previous step)
  // with chunk c+2 and the V slot of chunk c-1 with chunk c+1.
  const int n = nchunks;
  // key blocks of chunks c, c+1 and c+2 at step c; the next one is read from
  // the list during step c, so no list read sits between a step's barrier
  // and its copies
  auto block_of = [&](int c) { return (int)Ls[min(c, n - 1) / NCH]; };
  int jq0 = 0, jq1 = 0, jq2 = 0;
  auto step = [&](auto has_next, auto full, int c, const unsigned char* kS, const unsigned char* vP,
                  unsigned char* kI, unsigned char* vI, floatx16 (&sc)[NKT], floatx16 (&sn)[NKT]) {
    tile_barrier();
    if (c + 2 < n) issue_k(c + 2, jq2, kI);
    if (c + 1 < n) issue_v(c + 1, jq1, vI);
    const int jc = jq0;
    jq0 = jq1;
    jq1 = jq2;
    jq2 = block_of(c + 3);
    bf16x8 ring[KRD][NKT];
    if constexpr (decltype(has_next)::value) k_first(kS, ring);
    const float mc = prelude(c, jc, sc, decltype(full)::value);
    uint32_t pp[NP];
    // Two waves share each SIMD.  While one is in its S + softmax phase
    // (MFMAs interleaved with exp and convert work) it takes issue priority;
    // the other's PV phase, back-to-back MFMAs, keeps the matrix core busy
    // meanwhile.
    __builtin_amdgcn_s_setprio(1);
    s_and_p(has_next, std::true_type{}, kS, sn, sc, mc, pp, ring);
    __builtin_amdgcn_s_setprio(0);
    float lc = l_part;
    if constexpr (!decltype(full)::value)
      if (__builtin_amdgcn_ballot_w64(!(lc <= kChunkSumMax)) != 0) lc = raise_ref(sc, pp);
    l_run += lc;
    pv(pp, vP);
  };

  if (n > 0) {
    floatx16 sA[NKT], sB[NKT];
    uint32_t pp0[NP];
    jq0 = block_of(0);
    jq1 = block_of(1);
    jq2 = block_of(2);
    issue_k(0, jq0, kb0);
    issue_v(0, jq0, vb0);
    if (n > 1) issue_k(1, jq1, kb1);
    tile_barrier();
    {
      bf16x8 ring[KRD][NKT];
      k_first(kb0, ring);
      s_and_p(std::true_type{}, std::false_type{}, kb0, sA, sB, 0.f, pp0, ring);
    }
    // reference exponent: the first chunk's row max.  Key 0 of that chunk is
    // visible to every row (its block lies before the query block or is the
    // diagonal one), so the max is finite.
    causal_mask(0, jq0, sA);
    {
      const float mx = row_max(sA);
      mref = (mx == -INFINITY) ? 0.f : mx * scale_log2;
    }
    int c = 0;
    for (; c + 2 < n; c += 2) {
      step(std::true_type{}, std::false_type{}, c, kb1, vb0, kb0, vb1, sA, sB);
      step(std::true_type{}, std::false_type{}, c + 1, kb0, vb1, kb1, vb0, sB, sA);
    }
    // the last one or two steps raise the reference up front (`full`), as
    // they have no (or only a last) S work to hide a retry behind
    if (c + 1 < n) {
      step(std::true_type{}, std::true_type{}, c, kb1, vb0, kb0, vb1, sA, sB);
      step(std::false_type{}, std::true_type{}, c + 1, kb0, vb1, kb1, vb0, sB, sA);
    } else {
      step(std::false_type{}, std::true_type{}, c, kb1, vb0, kb0, vb1, sA, sB);
    }
  }

  // ---- epilogue: O = O^T / l, LSE.  The last step reads no K tile and every
  // wave has passed its barrier, so the staging regions are free again: the
  // wave writes its rows there (lane: 4 values of row lq at d0) and stores
  // them back as whole rows.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int t = i * BLK + qrow;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int slot = dt * 4 + rg;  // 16-byte slot of d0 = dt*32 + rg*8 (+ lg*4)
      *reinterpret_cast<uint2*>(stage + lq * ROWB + ((slot ^ kslot_x) * 16) + lg * 8) =
          make_uint2(pack_bf16x2(oacc[dt][rg * 4] * inv, oacc[dt][rg * 4 + 1] * inv),
                     pack_bf16x2(oacc[dt][rg * 4 + 2] * inv, oacc[dt][rg * 4 + 3] * inv));
    }
  // the region is this wave's alone: LDS serves a wave's accesses in order
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  char* odst = reinterpret_cast<char*>(O + row0);
  // the lane id afresh, so that no offset of the Q copies is kept (in
  // registers the main loop needs) until here
  const int le = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
  for (int m = 0; m < 32 / RPI; ++m) {
    const int r = m * RPI + le / SLOTS, sl = le % SLOTS;
    const uint4 w = *reinterpret_cast<const uint4*>(stage + r * ROWB + ((sl ^ k_swz<SLOTS>(r)) * 16));
    *reinterpret_cast<uint4*>(odst + row_ofs(r, sl)) = w;
  }
  if (LSE != nullptr && lg == 0)
    LSE[((size_t)b * Hq + h) * S + t] =
        l_tot > 0.f ? (mref + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int BLK, int KCH, int LMAX>
static hipError_t launch_direct(const void* q, const void* k, const void* v, const PrefillDims& d,
                                const int32_t* bidx, const int32_t* bcnt, float scale, void* out,
                                float* lse, hipStream_t st) {
  using Tr = DirectTraits<D, BLK, KCH>;
  auto kern = prefill_attn_bf16_kernel<D, BLK, KCH, LMAX>;
  if (d.S / BLK > LMAX) return hipErrorInvalidValue;
  const int units = d.B * d.Hkv * (d.S / BLK);
  const int grid = (units + kXcds - 1) / kXcds * kXcds * (d.Hq / d.Hkv);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Tr::NT), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), bidx, bcnt,
                     static_cast<uint16_t*>(out), lse, d.S, d.Hq, d.Hkv, scale * kLog2e, units);
  return hipGetLastError();
}

// Chunk size and list capacity per shape.  Blocks of 128 keys: 64-key chunks
// (about 73 KB of LDS, two 4-wave workgroups per CU).  Blocks of 64 keys have
// only two waves per workgroup, so their chunks are 32 keys: with a list of at
// most 2048 blocks (S <= 128K) a workgroup takes under 40 KB and four fit on a
// CU; longer prompts take the 4096-entry list and three.
template <int D>
static hipError_t launch_for_block(const void* q, const void* k, const void* v,
                                   const PrefillDims& d, const int32_t* bidx, const int32_t* bcnt,
                                   float scale, void* out, float* lse, hipStream_t st) {
  if (d.T == 128) return launch_direct<D, 128, 64, kMaxBlocks>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  if (d.T == 64 && d.S / 64 <= 2048)
    return launch_direct<D, 64, 32, 2048>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  if (d.T == 64) return launch_direct<D, 64, 32, kMaxBlocks>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_attn_bf16(const void* q, const void* k, const void* v,
                                    const PrefillDims& d, const int32_t* bidx,
                                    const int32_t* bcnt, float scale, void* out, float* lse,
                                    hipStream_t st) {
  if (d.D == 128) return launch_for_block<128>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  if (d.D == 64) return launch_for_block<64>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  return hipErrorInvalidValue;
}

hipError_t debug_flags_prefill_bf16(uint32_t* flags, bool clear) {
  return debug_flags_of_tu(flags, clear);
}

}  // namespace fsa
