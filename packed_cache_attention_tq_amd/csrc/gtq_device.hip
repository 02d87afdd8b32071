// GPU part of libgtq for gfx950: plan upload, the fused rotate+quantize+pack
// append kernel, query rotation, the split-K packed-cache attention kernel and
// the log-sum-exp merge with the inverse value rotation.
//
// Method: Block-GTQ page (abstract, 5th sentence: attention over packed caches
// without a decoded fp16 KV cache) and the TurboQuant pipeline diagram ("paper"
// column: norm, random rotation, per-coordinate Lloyd-Max quantization).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "gtq_internal.h"

using namespace gtq;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

union H8 {  // an MFMA f16 operand as a vector, dwords or one uint4
  half8 h;
  uint32_t u[4];
  uint4 v;
};

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

namespace {

// An opaque copy of a register value: lane swaps take their second operand this way,
// because handed the same value twice this compiler folds their two results into one.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

gtq_status hip_fail(hipError_t e, const char* what) {
  return fail(GTQ_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// ============================================================================
// Append: per token and KV head, for each key group and for the value vector:
//   nu = ||x|| (fp64 sum of squares, stored fp32), z = sqrt(d) * Pi * x / nu,
//   code_i = #{k : z_i >= t_k}; pack (TurboQuant diagram, "paper" column).
// Chunk path: one wave handles the up to 8 consecutive slots that a prompt chunk
// covers in one value block; the workgroup keeps the head's rotations (transposed)
// in LDS.
// ============================================================================

// Paged caches: position s of sequence seq lives in pool page table[seq * tstride +
// s / P] at s % P; a contiguous cache (table NULL) is slice (seq, h) of `capacity`.
struct PageMap {
  const int32_t* table;
  int32_t P, log2P, n_pages, tstride;  // P = 2^log2P tokens per page
};

// Flat token index of position s of (seq, KV head h) in the cache buffers, or -1 when
// the page is absent (a table entry outside [0, n_pages)).
__device__ inline int64_t token_index(const PageMap& m, int64_t capacity, int n_kv, int seq, int h, int64_t s) {
  if (!m.table) return ((int64_t)seq * n_kv + h) * capacity + s;
  const int pg = m.table[(int64_t)seq * m.tstride + (s >> m.log2P)];
  if (pg < 0 || pg >= m.n_pages) return -1;
  return ((int64_t)pg * n_kv + h) * m.P + (s & (m.P - 1));
}

struct AppendArgs {
  const DevHead* heads;  // this layer's heads [n_kv]
  const float* rot;
  const uint16_t* rsplit;  // split rotations (binary16 hi, lo)
  const DevCodebook* cb;
  uint32_t* k_codes;
  float* k_norms;
  uint32_t* v_codes;
  float* v_norms;
  const float* k;
  const float* v;
  const int32_t* seq_idx;
  const int64_t* slot;
  const int32_t* step_len;  // if set: token b goes to sequence b, slot step_len[b] - 1
  unsigned long long* overflow;
  int64_t capacity;
  int64_t n_tok;
  int64_t pos0;
  int32_t seq;
  int32_t batch;
  int32_t n_kv;
  int32_t k_words;
  int32_t v_bits;
  int32_t nc;  // norm-corrected stored norms: nu * sqrt(d) / ||C[code]||
  PageMap pm;
};

__device__ inline int quantize(float z, const float* thr, int n_thr) {
  int c = 0;
  for (int k = 0; k < n_thr; ++k) c += (z >= thr[k]) ? 1 : 0;
  return c;
}

// fp64 sum over the 64 lanes of a wave with lane moves that stay in the VALU: DPP row
// shifts inside each 16-lane row, then the gfx950 row swaps. Every lane gets the
// total (in a fixed order; the stored fp32 norm of the square root may differ from
// another summation order by at most one unit in the last place).
__device__ inline double dpp_f64(double v, int ctrl) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  switch (ctrl) {
    case 0: lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false); break;  // quad [1,0,3,2]
    case 1: lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false); break;  // quad [2,3,0,1]
    case 2: lo = __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, false); break; // row half mirror
    default: lo = __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, false); break; // row mirror
  }
  return __builtin_bit_cast(double, (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32));
}
__device__ inline double swap_f64(double v, bool x32) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t rl, rh;
  if (x32) {
    auto a = __builtin_amdgcn_permlane32_swap(lo, opaque(lo), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(hi, opaque(hi), false, false);
    rl = (threadIdx.x & 32) ? a[0] : a[1];
    rh = (threadIdx.x & 32) ? b[0] : b[1];
  } else {
    auto a = __builtin_amdgcn_permlane16_swap(lo, opaque(lo), false, false);
    auto b = __builtin_amdgcn_permlane16_swap(hi, opaque(hi), false, false);
    rl = (threadIdx.x & 16) ? a[0] : a[1];
    rh = (threadIdx.x & 16) ? b[0] : b[1];
  }
  return __builtin_bit_cast(double, (uint64_t)rl | ((uint64_t)rh << 32));
}
__device__ inline double wave_sum_f64_fast(double v) {
  v += dpp_f64(v, 0);  // pairs
  v += dpp_f64(v, 1);  // quads
  v += dpp_f64(v, 2);  // half rows (the mirror of a quad-uniform value is the other quad)
  v += dpp_f64(v, 3);  // rows
  v += swap_f64(v, false);
  v += swap_f64(v, true);
  return v;
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ============================================================================
// Chunk append as a rotation GEMM on the matrix cores (TurboQuant diagram, "paper"
// column: norm, rotation, per-coordinate quantization; Block-GTQ abstract, 5th
// sentence: one TQ-MSE instance per equal-rate group).
// Per token and vector (each key group, the value): nu = ||x|| in fp64, u = x / nu,
// z = sqrt(d) Pi u, code = #{k : z >= t_k}. The product Pi u runs as MFMA 16x16x32
// f16 on split operands: 16 Pi = P_hi + P_lo (plan tables) and 256 u = U_hi + U_lo
// (binary16 each); P_hi U_hi + P_hi U_lo + P_lo U_hi leaves out a 2^-22-relative term,
// so z carries fp32-grade error.
// A workgroup (8 waves) takes one KV head and one role (keys or values); wave w keeps
// the rotation operands of outputs 16 w .. 16 w + 15 (x all 128 inputs) in registers:
// the key groups' rotations form one block-diagonal matrix in record position order,
// so a tile may hold outputs of two groups (rate, dimension and record bit are per
// lane). The workgroup streams 32-token tiles through LDS: stage, norms, split,
// products and codes, pack and store.
// ============================================================================

constexpr int kAppWaves = 8;
constexpr int kAppThreads = 64 * kAppWaves;
constexpr int kAppTile = 32;          // tokens per tile (two MFMA row tiles)
constexpr int kAppPitch = 136;        // halves per A row (128 inputs + 8: no bank conflicts)

struct AppendGemmShared {
  _Float16 ua[2][kAppTile][kAppPitch];  // U_hi, U_lo in record position (key) or coordinate order
  uint32_t pk[kAppTile][16];          // packed key records of the tile
  uint32_t pv[4][128];                // packed value blocks of the tile (8 tokens each)
  float nu[kAppTile][5];              // fp32 norms per token: key groups 0..3, value 4
  float thr[5][16];                   // quantizer thresholds by rate
  float cen[5][16];                   // centroids by rate (norm-corrected variant)
  double nu64[kAppTile][5];           // fp64 norms (norm-corrected variant)
  double cs[kAppTile][5];             // sum of C[code]^2 per token and group (exact in fp64)
};

// Norm-corrected stored norm: nu sqrt(d) / sqrt(sum C[code]^2), evaluated in fp64. The
// sum is exact whatever the order (binary16 centroids, at most 128 terms), so only nu
// carries summation-order rounding.
__device__ inline float corrected_norm(double nu, double csum, int d) {
  return nu > 0.0 ? (float)(nu * sqrt((double)d) / sqrt(csum)) : 0.f;
}

// OR over the 16 lanes of a row: DPP row operations. update_dpp with bound_ctrl (every
// source lane of these patterns is inside the row) lets the compiler fuse each step
// into one v_or_b32_dpp.
__device__ inline uint32_t row_or_u32(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);   // quad [1,0,3,2]
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);   // quad [2,3,0,1]
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true);  // half-row mirror
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true);  // row mirror
  return v;
}

// fp64 sum over the 16 lanes of a row (one token): DPP row operations
__device__ inline double row_sum_f64(double v) {
  v += dpp_f64(v, 0);
  v += dpp_f64(v, 1);
  v += dpp_f64(v, 2);
  v += dpp_f64(v, 3);
  return v;
}

// Walsh-Hadamard transform (unnormalised, Sylvester order: H[i][j] = (-1)^popcount(i & j))
// of a 128-vector held one element per thread, element e by the thread with e = tid - t0
// for two whole waves starting at t0. Strides 1..32 move inside a wave; stride 64 goes
// through buf (128 floats of LDS). Every thread of the workgroup must call it (one
// barrier); only the 128 owners' results mean anything.
__device__ inline float wht128(float x, int e, bool owner, float* buf) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float y = __shfl_xor(x, m);
    x = (e & m) ? y - x : x + y;
  }
  if (owner) buf[e] = x;
  __syncthreads();
  if (owner) {
    const float y = buf[e ^ 64];
    x = (e & 64) ? y - x : x + y;
  }
  return x;
}
constexpr float kInvSqrt128 = 0.0883883461356163f;  // fp32 nearest to 1/sqrt(128)

// (at most 128 VGPRs, a few spilled: two workgroups per compute unit, so that one's
// barriers and LDS round trips overlap the other's work)
__global__ void __launch_bounds__(kAppThreads) __attribute__((amdgpu_waves_per_eu(4))) append_gemm_kernel(AppendArgs a) {
  __shared__ AppendGemmShared S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, n = lane & 15;
  // a one-dimensional grid of gx x n_kv x 2 workgroups: workgroup w takes KV head
  // w mod n_kv, and its first tile and role from w / n_kv. Consecutive workgroups go to
  // the eight accelerator dies (XCDs) in turn, so with n_kv a divisor or a multiple of 8
  // all workgroups of a head run on the same dies, and each die's L2 fetches only its
  // own heads' rotations.
  const int h = (int)(blockIdx.x % (unsigned)a.n_kv);
  const int wr = (int)(blockIdx.x / (unsigned)a.n_kv);
  const int gx = (int)(gridDim.x / (2u * (unsigned)a.n_kv));
  const int bx = wr % gx;
  const bool vrole = wr >= gx;
  const DevHead* __restrict__ hp = a.heads + h;
  const int n_groups = hp->n_groups;

  // ---- this wave's output tile: outputs 16 wave .. 16 wave + 15 (record positions of the
  //      key, coordinates of the value) over all 128 inputs in 4 steps of 32; lane (q, n)
  //      owns output p_out and its group's rate and dimension
  const int p_out = 16 * wave + n;
  int gp = 0;
  if (!vrole) {
#pragma unroll
    for (int gg = 1; gg < kMaxGroups; ++gg)
      if (gg < n_groups && p_out >= hp->pos_off[gg]) gp = gg;
  }
  const int rp = vrole ? a.v_bits : hp->rate[gp];
  const int dp = vrole ? kD : hp->dim[gp];
  // key record: the lane's code bit; a row's 16 outputs are one run of at most 64 bits
  // from the bit of output 16 wave (lane 0), inside words w0 .. w0 + 2
  const int bitp = vrole ? 0 : hp->bit_off[gp] + (p_out - hp->pos_off[gp]) * rp;
  const int w0 = __builtin_amdgcn_readfirstlane(bitp) >> 5;
  const int g_lo = __builtin_amdgcn_readfirstlane(gp), g_hi = __builtin_amdgcn_readlane(gp, 15);
  // rotation operands: lane (q, n) holds row p_out, inputs 32 s + 8q .. +7, hi and lo
  uint4 bh[4], bl[4];
  {
    const uint16_t* base = a.rsplit + (vrole ? hp->rsv_off : hp->rsk_off) + (size_t)p_out * kD + 8 * q;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bh[st] = *reinterpret_cast<const uint4*>(base + 32 * st);
      bl[st] = *reinterpret_cast<const uint4*>(base + kD * kD + 32 * st);
    }
  }
  if (tid < 80) {
    (&S.thr[0][0])[tid] = (&a.cb->t[0][0])[tid];
    (&S.cen[0][0])[tid] = (&a.cb->c[0][0])[tid];
  }
  // zero the A operands once (the pitch's pad columns are never read)
  for (int e = tid; e < 2 * kAppTile * kAppPitch / 8; e += kAppThreads)
    reinterpret_cast<uint4*>(&S.ua[0][0][0])[e] = make_uint4(0, 0, 0, 0);

  // ---- this thread's 8 inputs of a tile: token tau = tid >> 4 (one 16-lane row per
  //      token), columns c = (tid & 15) + 16 i
  const int tau = tid >> 4, sub = tid & 15;
  // packed to keep them out of the register budget: input i's source column in byte
  // i & 3 of colp[i >> 2], its key group in bits 2i, 2i + 1 of grpp
  uint32_t colp[2] = {0u, 0u}, grpp = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = sub + 16 * i;  // record position (keys) or coordinate (values)
    int col = c, g = 0;
    if (!vrole) {
#pragma unroll
      for (int gg = 1; gg < kMaxGroups; ++gg)
        if (gg < n_groups && c >= hp->pos_off[gg]) g = gg;
      col = hp->coord[c];
    }
    colp[i >> 2] |= (uint32_t)col << (8 * (i & 3));
    grpp |= (uint32_t)g << (2 * i);
  }
  auto src_col = [&](int i) { return (int)__builtin_amdgcn_ubfe(colp[i >> 2], 8 * (i & 3), 8); };
  auto grp_of = [&](int i) { return (int)__builtin_amdgcn_ubfe(grpp, 2 * i, 2); };
  // (head fields the tile loop needs are all read before it: the loop's global stores
  // could alias them, so reads inside it would be repeated and waited for on every tile)
  const int nd_store = (tid < kAppTile * kNS && tid % kNS < n_groups) ? hp->dim[tid % kNS] : 1;
  const float* src = vrole ? a.v : a.k;
  const int64_t s_begin = a.pos0 & ~(int64_t)(GTQ_VBLOCK - 1), s_end = a.pos0 + a.n_tok;
  const int64_t n_tiles = (s_end - s_begin + kAppTile - 1) / kAppTile;
  const size_t sh = (size_t)a.seq * a.n_kv + h;
  const int kw = a.k_words, vb = a.v_bits;
  // the thread's 8 inputs of a tile: unconditional loads (token 0 of the chunk stands in
  // for tokens outside it) whose validity is applied where they are used, so that the
  // next tile's loads stay in flight during this one
  auto load_tile = [&](int64_t tile, float (&xr)[8]) {
    const int64_t s = s_begin + tile * kAppTile + tau;
    const bool ok = tile < n_tiles && s >= a.pos0 && s < s_end;
    const size_t row = ok ? ((size_t)(s - a.pos0) * a.n_kv + h) * kD : (size_t)h * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i) xr[i] = src[row + src_col(i)];
    return ok;
  };
  float xr[8];
  bool xok = load_tile(bx, xr);
  using KArgsA = const __attribute__((address_space(4))) AppendArgs;
  KArgsA* const ka0 = (KArgsA*)__builtin_amdgcn_kernarg_segment_ptr();

  for (int64_t tile = bx; tile < n_tiles; tile += gx) {
    // the arguments the tile reads, loaded again in each tile rather than held in
    // registers across the loop
    KArgsA* kap = ka0;
    asm volatile("" : "+s"(kap));
    const AppendArgs& A = *(const AppendArgs*)kap;
    const int64_t ts = s_begin + tile * kAppTile;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = xok ? xr[i] : 0.f;
    xok = load_tile(tile + gx, xr);  // next tile, in flight during this one
    __syncthreads();                  // the previous tile's stores have read the buffers
    if (tid < kAppTile * 16) (&S.pk[0][0])[tid] = 0u;
    (&S.pv[0][0])[tid] = 0u;          // 4 x 128 == kAppThreads
    if (A.nc && tid < kAppTile * 5) (&S.cs[0][0])[tid] = 0.0;
    // ---- norms (fp64, per token and group; every lane of the row gets all sums), then
    //      u = x / nu split as 256 u = U_hi + U_lo
    double sg[kMaxGroups] = {0.0, 0.0, 0.0, 0.0};
    if (vrole) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sg[0] = fma((double)x[i], (double)x[i], sg[0]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double xv = x[i];
#pragma unroll
        for (int gg = 0; gg < kMaxGroups; ++gg) sg[gg] += (grp_of(i) == gg) ? xv * xv : 0.0;
      }
    }
    // every lane gets each group's sum; the stored norm is the correctly rounded fp64
    // sqrt (lane sub computes group sub's), the scaling 1 / nu takes the hardware
    // reciprocal square root and one Newton step (relative error far below the split
    // products' 2^-22)
    const int ng = vrole ? 1 : n_groups;
    double inv[kMaxGroups], own = 0.0;
#pragma unroll
    for (int gg = 0; gg < kMaxGroups; ++gg) {
      inv[gg] = 0.0;
      if (gg < ng) {
        const double t = row_sum_f64(sg[gg]);
        if (sub == gg) own = t;
        if (t > 0.0) {
          const double y = __builtin_amdgcn_rsq(t);
          inv[gg] = y * fma(-0.5 * t, y * y, 1.5);
        }
      }
    }
    if (sub < ng) {
      const double nu = sqrt(own);
      S.nu[tau][vrole ? 4 : sub] = (float)nu;
      if (A.nc) S.nu64[tau][vrole ? 4 : sub] = nu;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double iv = inv[0];
#pragma unroll
      for (int gg = 1; gg < kMaxGroups; ++gg) iv = (grp_of(i) == gg) ? inv[gg] : iv;
      const float u = (float)((double)x[i] * iv) * 256.f;
      const _Float16 hi = (_Float16)u;
      S.ua[0][tau][sub + 16 * i] = hi;
      S.ua[1][tau][sub + 16 * i] = (_Float16)(u - (float)hi);
    }
    __syncthreads();
    // ---- products, codes and packing of this wave's tile (both 16-token halves)
    floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      H8 ph, pl;
      ph.v = bh[st];
      pl.v = bl[st];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        H8 ah, al;
        ah.v = *reinterpret_cast<const uint4*>(&S.ua[0][16 * hf + n][32 * st + 8 * q]);
        al.v = *reinterpret_cast<const uint4*>(&S.ua[1][16 * hf + n][32 * st + 8 * q]);
        acc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah.h, ph.h, acc[hf], 0, 0, 0);
        acc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al.h, ph.h, acc[hf], 0, 0, 0);
        acc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah.h, pl.h, acc[hf], 0, 0, 0);
      }
    }
    // lane (q, n) holds D[token 16 hf + 4q + e][output p_out]
    const float zs = sqrtf((float)dp) * (1.f / (kRotSplitScale * 256.f));
    const float* th = S.thr[rp];
    // code = #{k : z >= t_k} by binary search over the sorted thresholds of the lane's
    // rate, one search level at a time for all 8 values of the lane (the threshold reads
    // of a level go out together)
    int cds[8];
    float zv[8];
#pragma unroll
    for (int v8 = 0; v8 < 8; ++v8) {
      zv[v8] = acc[v8 >> 2][v8 & 3] * zs;
      cds[v8] = 0;
    }
#pragma unroll
    for (int lvl = 3; lvl >= 0; --lvl) {
      if (lvl < rp) {
        const int step = 1 << lvl;
        float tv[8];
#pragma unroll
        for (int v8 = 0; v8 < 8; ++v8) tv[v8] = th[cds[v8] + step - 1];
#pragma unroll
        for (int v8 = 0; v8 < 8; ++v8) cds[v8] += zv[v8] >= tv[v8] ? step : 0;
      }
    }
    if (A.nc) {
      // sum of C[code]^2 over each group's outputs in the row, for each of the lane's 8
      // tokens (the row's groups are g_lo .. g_hi)
      const float* cr = S.cen[rp];
#pragma unroll
      for (int v8 = 0; v8 < 8; ++v8) {
        const double c = (double)cr[cds[v8]];
        for (int g = g_lo; g <= g_hi; ++g) {
          const double rs = row_sum_f64(gp == g ? c * c : 0.0);
          if (n == 0) atomicAdd(&S.cs[16 * (v8 >> 2) + 4 * q + (v8 & 3)][vrole ? 4 : g], rs);
        }
      }
    }
    if (vrole) {
      const int r = rp, i = p_out;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cd = cds[4 * hf + e];
          const int t = 16 * hf + 4 * q + e;
          // token t & 7 of block t >> 3, coordinate i at bit 8 vb i + vb (t & 7)
          const int bit = 8 * r * i + r * (t & 7);
          uint32_t* dst = &S.pv[t >> 3][0];
          const uint64_t f = (uint64_t)cd << (bit & 31);
          atomicOr(dst + (bit >> 5), (uint32_t)f);
          if (f >> 32) atomicOr(dst + (bit >> 5) + 1, (uint32_t)(f >> 32));
        }
      }
    } else {
      // keys: each lane places its code in the row's 96-bit window from word w0, the row
      // ORs the window together and three lanes OR its words into the record
      const int pos = bitp - 32 * w0;
      const int kq = pos >> 5, sft = pos & 31;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cd = cds[4 * hf + e];
          const uint32_t lo = (uint32_t)cd << sft;
          const uint32_t hi = sft ? (uint32_t)cd >> (32 - sft) : 0u;
          uint32_t v0 = kq == 0 ? lo : 0u;
          uint32_t v1 = kq == 0 ? hi : (kq == 1 ? lo : 0u);
          uint32_t v2 = kq == 1 ? hi : (kq == 2 ? lo : 0u);
          v0 = row_or_u32(v0);
          v1 = row_or_u32(v1);
          v2 = row_or_u32(v2);
          const int t = 16 * hf + 4 * q + e;
          const uint32_t vv = n == 0 ? v0 : (n == 1 ? v1 : v2);
          if (n < 3 && vv) atomicOr(&S.pk[t][w0 + n], vv);
        }
      }
    }
    __syncthreads();
    // ---- store (thread indices from an opaque copy: the store addresses are derived
    //      here rather than held, or spilled, across the tile)
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o;
    if (!vrole) {
      for (int e = tid; e < kAppTile * kw; e += kAppThreads) {
        const int t = e / kw, w = e - t * kw;
        const int64_t s = ts + t;
        if (s >= A.pos0 && s < s_end) {
          const int64_t ti = token_index(A.pm, A.capacity, A.n_kv, A.seq, h, s);
          if (ti >= 0) A.k_codes[ti * kw + w] = S.pk[t][w];
        }
      }
      if (tid < kAppTile * kNS) {
        const int t = tid / kNS, g = tid - kNS * t;
        const int64_t s = ts + t;
        if (s >= A.pos0 && s < s_end) {
          const int64_t ti = token_index(A.pm, A.capacity, A.n_kv, A.seq, h, s);
          if (ti >= 0)
            A.k_norms[ti * kNS + g] =
                g >= n_groups ? 0.f : (A.nc ? corrected_norm(S.nu64[t][g], S.cs[t][g], nd_store) : S.nu[t][g]);
          else if (g == 0 && h == 0)
            atomicAdd(A.overflow, 1ull);  // once per token in an absent page
        }
      }
    } else {
      const int vw = 32 * vb;
      for (int e = tid; e < 4 * vw; e += kAppThreads) {
        const int b = e / vw, w = e - b * vw;
        const int64_t sb = ts + 8 * b;
        if (sb + 8 <= A.pos0 || sb >= s_end) continue;  // no token of this block in the chunk
        const int64_t bi = token_index(A.pm, A.capacity, A.n_kv, A.seq, h, sb);  // (8-aligned: a block index x 8)
        if (bi < 0) continue;
        uint32_t* blk = A.v_codes + (size_t)(bi / GTQ_VBLOCK) * vw;
        if (sb >= A.pos0 && sb + 8 <= s_end) {
          blk[w] = S.pv[b][w];
        } else {
          // bits of the block's tokens inside the chunk only
          uint32_t mask = 0;
          for (int jt = 0; jt < 8; ++jt) {
            if (sb + jt < A.pos0 || sb + jt >= s_end) continue;
            const int c_lo = (32 * w) / (8 * vb), c_hi = min(kD - 1, (32 * w + 31) / (8 * vb));
            for (int cc = c_lo; cc <= c_hi; ++cc) {
              const int bit = 8 * vb * cc + vb * jt - 32 * w;
              const uint32_t m = (1u << vb) - 1u;
              if (bit >= 0 && bit < 32) mask |= m << bit;
              else if (bit < 0 && bit > -vb) mask |= m >> (-bit);
            }
          }
          if (mask) {
            atomicAnd(blk + w, ~mask);
            atomicOr(blk + w, S.pv[b][w] & mask);
          }
        }
      }
      if (tid < kAppTile) {
        const int64_t s = ts + tid;
        const int64_t ti = (s >= A.pos0 && s < s_end) ? token_index(A.pm, A.capacity, A.n_kv, A.seq, h, s) : -1;
        if (ti >= 0) A.v_norms[ti] = A.nc ? corrected_norm(S.nu64[tid][4], S.cs[tid][4], kD) : S.nu[tid][4];
      }
    }
  }
}

// One workgroup (1024 threads) per (token, KV head) doing everything (role 3), or, when
// few tokens leave most of the chip idle, three per (token, KV head), one per role: the
// key (role 0), value coordinates 0..63 (role 1) and 64..127 (role 2), so that each
// loads a third of the rotation rows; a value rotation that needs all 128 coordinates
// at once (a Hadamard transform, or the norm-corrected sum over all codes) stays in
// role 1.
// All global loads go out in one round (the vectors in natural order, the rotation rows
// each thread needs, the token's sequence and slot); the key is put in record order in
// LDS; the norms are fp64 wave reductions; thread (output o, quarter qq) forms a
// quarter of one rotated coordinate. The two value halves write disjoint words of the
// token's value block.
// A head's key group layout, read in one round of uniform loads (none waits on another;
// short-circuit tests on n_groups would chain them), and selection by group index
// without indexed (per-lane) loads.
struct GroupLayout {
  int n;
  int pos[kMaxGroups], dim[kMaxGroups], rate[kMaxGroups], bit[kMaxGroups], kp[kMaxGroups];
  int64_t krot[kMaxGroups];
};
// (written out without loops: every array index is a constant from the start, so the
// struct lives in registers)
static_assert(kMaxGroups == 4, "the layout helpers are written for four groups");
__device__ inline GroupLayout load_layout(const DevHead* hd) {
  GroupLayout L;
  L.n = hd->n_groups;
  L.pos[0] = hd->pos_off[0], L.pos[1] = hd->pos_off[1], L.pos[2] = hd->pos_off[2], L.pos[3] = hd->pos_off[3];
  L.dim[0] = hd->dim[0], L.dim[1] = hd->dim[1], L.dim[2] = hd->dim[2], L.dim[3] = hd->dim[3];
  L.rate[0] = hd->rate[0], L.rate[1] = hd->rate[1], L.rate[2] = hd->rate[2], L.rate[3] = hd->rate[3];
  L.bit[0] = hd->bit_off[0], L.bit[1] = hd->bit_off[1], L.bit[2] = hd->bit_off[2], L.bit[3] = hd->bit_off[3];
  L.kp[0] = hd->kp_off[0], L.kp[1] = hd->kp_off[1], L.kp[2] = hd->kp_off[2], L.kp[3] = hd->kp_off[3];
  L.krot[0] = hd->krot_off[0], L.krot[1] = hd->krot_off[1], L.krot[2] = hd->krot_off[2], L.krot[3] = hd->krot_off[3];
  return L;
}
// group of record position p
__device__ inline int group_of(const GroupLayout& L, int p) {
  int g = 0;
  g = (1 < L.n && p >= L.pos[1]) ? 1 : g;
  g = (2 < L.n && p >= L.pos[2]) ? 2 : g;
  g = (3 < L.n && p >= L.pos[3]) ? 3 : g;
  return g;
}
template <typename T>
__device__ inline T pick(const T (&v)[kMaxGroups], int g) {
  return g == 3 ? v[3] : (g == 2 ? v[2] : (g == 1 ? v[1] : v[0]));
}

__device__ __attribute__((always_inline)) inline void append_token_body(const AppendArgs& a, int64_t tok, int h, int role) {
  __shared__ float xnat[2 * kD];        // key then value, natural order
  __shared__ __align__(16) float xs[2 * kD];  // key (record order) then value coordinates
  __shared__ float red[4][2 * kD];
  __shared__ float nu_s[5], sc_s[5];
  __shared__ double nu64_s[5], cs_s[5];  // norm-corrected variant: fp64 norms, sums of C[code]^2
  __shared__ uint32_t krec[16];
  __shared__ uint32_t vblk[128], vmask[128];
  __shared__ float kcen[kD];            // QJL: the decoded centroid of each key record position
  __shared__ double rnat[kD];           // QJL: the residual in head coordinates
  __shared__ float thr[5][16], cen[5][16];
  const int tid = threadIdx.x;
  const DevHead* __restrict__ hd = a.heads + h;
  const GroupLayout GL = load_layout(hd);
  const int n_groups = GL.n;
  const size_t row = ((size_t)tok * a.n_kv + h) * kD;
  float xv = 0.f;
  if (tid < kD) xv = a.k[row + tid];
  else if (tid < 2 * kD) xv = a.v[row + tid - kD];
  const int crd = tid < kD ? hd->coord[tid] : 0;
  const float thv = tid < 80 ? (&a.cb->t[0][0])[tid] : 0.f;
  const float cev = tid < 80 ? (&a.cb->c[0][0])[tid] : 0.f;
  // this thread's rotation entries: key output o < 128 (row i of its group, pair range
  // of quarter qq) or value output o - 128 (32 columns of quarter qq), if its role's
  const int o = tid & 255, qq = tid >> 8;
  const bool vsplit = !a.nc && !hd->v_hadamard;
  const int vlo = role == 2 ? kD / 2 : 0, vhi = (role == 1 && vsplit) ? kD / 2 : kD;
  const bool mine = role == 3 || (role == 0 ? o < kD : (o >= kD + vlo && o < kD + vhi));
  const bool do_k = role == 0 || role == 3, do_v = role != 0;
  // (key: column pairs klo + 2u and klo + 2u + 1 in rv[u]; value: columns 32 qq + 4u ..)
  float4 rv[8];
  int kg = 0, klo = 0, khi = 0;
  if (o < kD) {
    kg = group_of(GL, o);
    const int d = pick(GL.dim, kg), i = o - pick(GL.pos, kg), dp = d >> 1;
    klo = (dp * qq) >> 2;
    khi = (dp * (qq + 1)) >> 2;
    if (!mine) khi = klo;  // (no key work outside role 0)
    const float2* pr = reinterpret_cast<const float2*>(a.rot + pick(GL.krot, kg) + (size_t)i * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float2 p0 = (klo + 2 * u < khi) ? pr[klo + 2 * u] : make_float2(0.f, 0.f);
      const float2 p1 = (klo + 2 * u + 1 < khi) ? pr[klo + 2 * u + 1] : make_float2(0.f, 0.f);
      rv[u] = make_float4(p0.x, p0.y, p1.x, p1.y);
    }
  } else {
    const float4* pr = reinterpret_cast<const float4*>(a.rot + hd->vrot_off + (size_t)(o - kD) * kD + 32 * qq);
#pragma unroll
    for (int u = 0; u < 8; ++u) rv[u] = (hd->v_hadamard || !mine) ? make_float4(0.f, 0.f, 0.f, 0.f) : pr[u];
  }
  // (a chunk through this kernel: no index arrays, token tok of sequence a.seq at pos0 + tok)
  const int seq = a.step_len ? (int)tok : (a.seq_idx ? a.seq_idx[tok] : a.seq);
  const int64_t slot = a.step_len ? (int64_t)a.step_len[tok] - 1 : (a.slot ? a.slot[tok] : a.pos0 + tok);
  const int64_t ti = (seq < 0 || seq >= a.batch || slot < 0 || slot >= a.capacity)
                         ? -1 : token_index(a.pm, a.capacity, a.n_kv, seq, h, slot);
  if (ti < 0) {
    if (tid == 0 && h == 0 && do_k) atomicAdd(a.overflow, 1ull);  // once per token
    return;
  }
  if (role == 2 && !vsplit) return;  // role 1 does the whole value
  if (tid < 2 * kD) xnat[tid] = xv;
  if (tid < 80) {
    (&thr[0][0])[tid] = thv;
    (&cen[0][0])[tid] = cev;
  }
  if (tid < 5) cs_s[tid] = 0.0;
  if (tid < 16) krec[tid] = 0u;
  if (tid < 128) {
    vblk[tid] = 0u;
    vmask[tid] = 0u;
  }
  __syncthreads();
  if (tid < kD) xs[tid] = xnat[crd];
  else if (tid < 2 * kD) xs[tid] = xnat[tid];
  __syncthreads();
  // norms: wave 0 the key groups (all four sums at once), wave 1 the value vector
  if (tid < 64) {
    const double x0 = xs[2 * tid], x1 = xs[2 * tid + 1];
    const double sq = x0 * x0 + x1 * x1;
    const int mg = group_of(GL, 2 * tid);
    double s4[kMaxGroups];
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) s4[g] = (mg == g) ? sq : 0.0;
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) s4[g] = wave_sum_f64_fast(s4[g]);
    if (tid < n_groups) {  // lane g finishes group g (every lane holds all four sums)
      double sg = s4[0];
#pragma unroll
      for (int g = 1; g < kMaxGroups; ++g) sg = (tid == g) ? s4[g] : sg;
      const double nu = sqrt(sg);
      nu_s[tid] = (float)nu;
      nu64_s[tid] = nu;
      sc_s[tid] = nu > 0.0 ? (float)(sqrt((double)pick(GL.dim, tid)) / nu) : 0.f;
    }
  } else if (tid < 128) {
    const int l = tid - 64;
    const double x0 = xs[kD + 2 * l], x1 = xs[kD + 2 * l + 1];
    const double s = wave_sum_f64_fast(x0 * x0 + x1 * x1);
    if (l == 0) {
      const double nu = sqrt(s);
      nu_s[4] = (float)nu;
      nu64_s[4] = nu;
      sc_s[4] = nu > 0.0 ? (float)(sqrt((double)kD) / nu) : 0.f;
    }
  }
  // rotation partial sums
  {
    float acc = 0.f;
    if (o < kD) {
      const float2* x = reinterpret_cast<const float2*>(xs + pick(GL.pos, kg));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (klo + 2 * u < khi) {
          const float2 xx = x[klo + 2 * u];
          acc = fmaf(rv[u].x, xx.x, acc);
          acc = fmaf(rv[u].y, xx.y, acc);
        }
        if (klo + 2 * u + 1 < khi) {
          const float2 xx = x[klo + 2 * u + 1];
          acc = fmaf(rv[u].z, xx.x, acc);
          acc = fmaf(rv[u].w, xx.y, acc);
        }
      }
    } else if (!hd->v_hadamard) {
      const float* x = xs + kD + 32 * qq;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc = fmaf(rv[u].x, x[4 * u], acc);
        acc = fmaf(rv[u].y, x[4 * u + 1], acc);
        acc = fmaf(rv[u].z, x[4 * u + 2], acc);
        acc = fmaf(rv[u].w, x[4 * u + 3], acc);
      }
    }
    red[qq][o] = acc;
  }
  if (hd->v_hadamard) {  // Pi_V v = c H (s * v): threads 128..255 own coordinate tid - 128
    __shared__ float hbuf[kD];
    const bool owner = tid >= kD && tid < 2 * kD;
    const int e = tid - kD;
    const float x = owner ? hd->vsign[e] * xs[kD + e] : 0.f;
    const float y = wht128(x, e & (kD - 1), owner, hbuf);
    if (owner) red[0][tid] = y * kInvSqrt128;
  }
  __syncthreads();
  const int vb = a.v_bits;
  const int j0 = (int)(slot & (GTQ_VBLOCK - 1));
  const bool qown = tid < kD ? do_k : (do_v && tid >= kD + vlo && tid < kD + vhi);
  if (tid < 2 * kD && qown) {  // (whole waves: 0-1 keys, 2 and/or 3 values)
    const float z0 = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    if (tid < kD) {
      const int g = kg;
      const int b = pick(GL.rate, g);
      const uint32_t c = quantize(z0 * sc_s[g], thr[b], (1 << b) - 1);
      kcen[tid] = cen[b][c];
      const int bit = pick(GL.bit, g) + (tid - pick(GL.pos, g)) * b;
      const uint64_t f = (uint64_t)c << (bit & 31);
      atomicOr(&krec[bit >> 5], (uint32_t)f);
      if (f >> 32) atomicOr(&krec[(bit >> 5) + 1], (uint32_t)(f >> 32));
      if (a.nc) {  // per-group sums of C[code]^2 (waves 0 and 1 hold the key outputs)
        const double c2 = (double)cen[b][c] * (double)cen[b][c];
        double s4[kMaxGroups];
#pragma unroll
        for (int gg = 0; gg < kMaxGroups; ++gg) s4[gg] = wave_sum_f64_fast(g == gg ? c2 : 0.0);
        if ((tid & 63) < n_groups) {
          double sv = s4[0];
#pragma unroll
          for (int gg = 1; gg < kMaxGroups; ++gg) sv = ((tid & 63) == gg) ? s4[gg] : sv;
          atomicAdd(&cs_s[tid & 63], sv);
        }
      }
    } else {
      const int cidx = tid - kD;
      const uint32_t c = quantize(z0 * sc_s[4], thr[vb], (1 << vb) - 1);
      if (a.nc) {
        const double c2 = wave_sum_f64_fast((double)cen[vb][c] * (double)cen[vb][c]);
        if ((tid & 63) == 0) atomicAdd(&cs_s[4], c2);
      }
      const int bit = 8 * vb * cidx + vb * j0;
      const uint64_t f = (uint64_t)c << (bit & 31);
      const uint64_t m = (uint64_t)((1u << vb) - 1u) << (bit & 31);
      atomicOr(&vblk[bit >> 5], (uint32_t)f);
      atomicOr(&vmask[bit >> 5], (uint32_t)m);
      if (m >> 32) {
        atomicOr(&vblk[(bit >> 5) + 1], (uint32_t)(f >> 32));
        atomicOr(&vmask[(bit >> 5) + 1], (uint32_t)(m >> 32));
      }
    }
  }
  __syncthreads();
  if (hd->qjl && do_k) {
    // 1-bit QJL residual sketch (TurboQuant-prod; diagram residual and QJL boxes): the
    // decoded key k_hat (stored norms), r = k - k_hat and gamma = |r| in fp64, then
    // sign(S r) into record words mse .. mse + 3 and gamma's fp32 bits into mse + 4.
    // Thread (record position p, eighth e) sums its sixteenth of column p of Pi_g.
    const int p = tid >> 3, e = tid & 7;
    const int g = group_of(GL, p);
    const int d = pick(GL.dim, g), po = pick(GL.pos, g), ii = p - po;
    const float* col = a.rot + pick(GL.krot, g) + ii;
    double s = 0.0;
    for (int i = 16 * e; i < min(d, 16 * e + 16); ++i) s += (double)col[(size_t)i * d] * (double)kcen[po + i];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    const double nu = a.nc ? (double)corrected_norm(nu64_s[g], cs_s[g], d) : (double)nu_s[g];
    const double r = (double)xs[p] - nu * (s / sqrt((double)d));
    if (e == 0) rnat[hd->coord[p]] = r;
    __syncthreads();
    // gamma: threads 0..127 take the residual's coordinate tid
    __shared__ double gsum[2];
    if (tid < kD) {
      const double w = wave_sum_f64_fast(rnat[tid] * rnat[tid]);
      if ((tid & 63) == 0) gsum[tid >> 6] = w;
    }
    // projections: thread (row j, eighth e) sums its sixteenth of row j of S
    const float4* srow = reinterpret_cast<const float4*>(a.rot + hd->qjl_off + (size_t)p * kD + 16 * e);
    double pj = 0.0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 sv = srow[u];
      pj += (double)sv.x * rnat[16 * e + 4 * u] + (double)sv.y * rnat[16 * e + 4 * u + 1] +
            (double)sv.z * rnat[16 * e + 4 * u + 2] + (double)sv.w * rnat[16 * e + 4 * u + 3];
    }
    pj += __shfl_xor(pj, 1);
    pj += __shfl_xor(pj, 2);
    pj += __shfl_xor(pj, 4);
    // bits j of the wave (lanes with e == 0): 8 per wave, 32 per word
    const unsigned long long bal = __ballot(e == 0 && pj >= 0.0);
    __shared__ uint32_t sbits[16];  // (1024 threads: 16 waves)
    if ((tid & 63) == 0) {
      uint32_t b8 = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) b8 |= (uint32_t)((bal >> (8 * k)) & 1ull) << k;
      sbits[tid >> 6] = b8;
    }
    __syncthreads();
    const int mw = hd->mse_words;
    if (tid < 4) krec[mw + tid] = sbits[4 * tid] | sbits[4 * tid + 1] << 8 | sbits[4 * tid + 2] << 16 | sbits[4 * tid + 3] << 24;
    if (tid == 4) krec[mw + 4] = __builtin_bit_cast(uint32_t, (float)sqrt(gsum[0] + gsum[1]));
    __syncthreads();
  }
  if (do_k && tid < a.k_words) a.k_codes[ti * a.k_words + tid] = krec[tid];
  if (do_k && tid >= 64 && tid < 64 + kNS) {
    const int g = tid - 64;
    a.k_norms[ti * kNS + g] =
        g >= n_groups ? 0.f : (a.nc ? corrected_norm(nu64_s[g], cs_s[g], pick(GL.dim, g)) : nu_s[g]);
  }
  if ((role == 1 || role == 3) && tid == 128) a.v_norms[ti] = a.nc ? corrected_norm(nu64_s[4], cs_s[4], kD) : nu_s[4];
  if (do_v && tid >= 256 && tid < 256 + 32 * vb) {
    const int w = tid - 256;
    const uint32_t m = vmask[w];
    if (m) {
      uint32_t* blk = a.v_codes + (size_t)(ti / GTQ_VBLOCK) * (32 * vb);  // (slices hold whole blocks)
      atomicAnd(blk + w, ~m);
      atomicOr(blk + w, vblk[w] & m);
    }
  }
}

// grid (tokens, KV heads, 1 or 3 roles)
__global__ void __launch_bounds__(1024) append_token_kernel(AppendArgs a) {
  append_token_body(a, blockIdx.x, blockIdx.y, gridDim.z == 1 ? 3 : (int)blockIdx.z);
}

// roles per (token, KV head) of the per-token append: 3 while n token-heads leave most of
// the compute units idle, else 1
inline int append_roles(int64_t n_token_heads) { return n_token_heads < 128 ? 3 : 1; }

// ============================================================================
// Split-K attention over the packed cache (Block-GTQ page, abstract, 5th
// sentence), in three launches:
//   attn_qrot_kernel      r_g = Pi_g q_g for every key group and query row, scaled by
//                         scale / sqrt(d_g) * log2(e) and split into a binary16 high part
//                         and a binary16 remainder (together ~22 bits): the QK B operand
//                         of each row tile (columns 0..7: high parts of rows 0..7,
//                         columns 8..15: low parts of rows 7..0), kept in the workspace;
//   attn_partials_kernel  per (row tile, split of `chunk` tokens) one online-softmax
//                         partial (m, l, acc[128]) per row;
//   attn_merge_tile_kernel / attn_merge_kernel
//                         log-sum-exp merge of the splits and o = Pi_V^T acc / sqrt(128).
// Partials: a workgroup (8 waves) takes one row tile (up to 8 query rows of one sequence
// and KV head) and one split; each wave walks 32-token blocks, staging each block in its
// LDS area and issuing the next block's loads before computing on the stage:
//   QK: per 32-coordinate K-block (one rate and key group each; their count is a
//       template parameter, so the loop is straight-line) one MFMA 16x16x32 f16 per
//       16-token half; A = decoded key codes (exact binary16 codebook values, two codes
//       per table read), B = the rotated queries. The per-token group norm multiplies
//       each product; a row-mirror DPP then adds the high and low halves.
//   online softmax in base 2 (the scale carries log2(e)), each of the two lanes of a
//       row pair finishing four of the eight tokens;
//   PV: MFMA with A = p * nu_V split into high/low parts (rows as above) and
//       B = decoded value codes (8 tokens x 16 coordinates), accumulating in the value
//       rotation's basis.
// The waves merge through LDS into one partial per row.
// ============================================================================

constexpr float kPvLimit = 16384.f;  // p * nu_V <= 2^14 keeps the binary16 high parts finite
constexpr int kWaves = 8;          // waves per partials workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kPS = 132;           // partial record: m, l, 2 pad, acc[128] (16-byte aligned acc)
constexpr int kMaxChunks = 256;    // splits per row
constexpr int kQB = kMaxKB * 64;   // uint4 entries of a tile's QK B operand (8 KB)
constexpr int kTargetWG = 256;     // partials workgroups the automatic split aims at

struct AttnArgs {
  const DevHead* heads;
  const float* rot;
  const DevCodebook* cb;
  const uint32_t* k_codes;
  const float* k_norms;
  const uint32_t* v_codes;
  const float* v_norms;
  const float* q;          // [rows][128] (rotation only)
  float* logits;           // decode only, optional
  const int32_t* seq_len;  // decode
  uint4* qb;               // [tiles][kQB] QK B operands
  float* tile_xs;          // [tiles]: 2^sq, the factor that undoes the operands' range scaling
  uint4* qjl_qb;           // QJL plans: [tiles][4 * 64] B operands of the residual sketch (S q)
  int32_t qjl, mse_words;  // QJL plan; words of a key record's MSE part
  float* partials;         // [rows][n_chunks][kPS]
  int64_t capacity;
  int64_t logits_ld;
  int64_t pos0;            // prefill
  int32_t n_kv, n_q, g, k_words;
  int32_t tiles_per_kv;    // row tiles per KV head (8 rows per tile in decode, 16 in prefill)
  int32_t prefill;         // 0 decode, 1 prefill
  int32_t seq;             // prefill sequence
  int32_t n_tok;           // prefill: tokens in chunk
  int32_t chunk;           // tokens per split (multiple of 32)
  int32_t n_chunks;
  int32_t max_len;         // decode clamp
  int32_t nkb_max;         // largest K-block count of the layer's heads
  float qscale;            // softmax scale * log2(e)
  // fp16 sink and recent-token buffers (decode only): their split is the last one
  const uint16_t* wk_sink;
  const uint16_t* wv_sink;
  const uint16_t* wk_rec;
  const uint16_t* wv_rec;
  int32_t win;             // 1: split n_chunks - 1 is the fp16 window's
  int32_t n_sink, sink_slots, n_recent;
  PageMap pm;              // paged cache (pm.table set) or contiguous
  // decode: the partials kernel's workgroups (sk_G) share the (tile, 32-token block)
  // units of the batch equally; partial record of segment s (workgroup w on tile t:
  // s = w + t; the window split of tile t: s = sk_G + n_tiles + t), row r of the tile:
  // partials + (8 s + r) kPS
  int32_t batch, n_tiles, sk_G;
  // decode: per row tile, written by the workgroup that runs its first block: (first
  // workgroup w0 on it, its number of workgroups, all units low and high 32 bits)
  int4* tile_info;
};

// End of the packed positions of a sequence of length L with n_sink sink and n_recent
// recent fp16 positions: the packed ones are [n_sink, packed_end).
__host__ __device__ inline int packed_end(int L, int n_sink, int n_recent) {
  return L > n_sink + n_recent ? L - n_recent : min(L, n_sink);
}

// Decode work units: the 32-token blocks of each row tile's packed range (every tile of a
// sequence has the sequence's length). Workgroup w of G takes units [w U / G, (w + 1) U / G).
__device__ inline int seq_blocks(const int32_t* seq_len, int b, int max_len, int win, int n_sink, int n_recent) {
  int L = min(max(seq_len[b], 0), max_len);
  if (win) L = packed_end(L, n_sink, n_recent);
  return (L + 31) >> 5;
}
// the workgroup whose range holds unit u (0 <= u < U)
__device__ inline int sk_owner(int64_t u, int G, int64_t U) { return (int)(((u + 1) * G - 1) / U); }
// whether workgroup w has units (with fewer units than workgroups some have none, and
// write no partial)
__device__ inline bool sk_live(int64_t w, int G, int64_t U) { return (w + 1) * U / G > w * U / G; }

// tile -> (sequence, KV head, tile within the head)
__device__ inline void tile_coords(const AttnArgs& a, int tile, int* seq, int* h, int* tr) {
  if (a.prefill) {
    *h = tile / a.tiles_per_kv;
    *tr = tile - *h * a.tiles_per_kv;
    *seq = a.seq;
  } else {
    *seq = tile / (a.n_kv * a.tiles_per_kv);
    const int rem = tile - *seq * a.n_kv * a.tiles_per_kv;
    *h = rem / a.tiles_per_kv;
    *tr = rem - *h * a.tiles_per_kv;
  }
}

// query row r (0..RT-1) of a tile of RT rows: its global row id (-1 if absent) and
// visible length
template <int RT = 8>
__device__ inline int tile_row(const AttnArgs& a, int seq, int h, int tr, int r, int len_ld, int* len) {
  const int f = tr * RT + r;
  int id = -1, L = 0;
  if (a.prefill) {
    if (f < a.n_tok * a.g) {
      const int t = f / a.g;
      id = t * a.n_q + h * a.g + (f - t * a.g);
      L = (int)(a.pos0 + t + 1);
    }
  } else if (f < a.g) {
    id = seq * a.n_q + h * a.g + f;
    L = min(max(len_ld, 0), a.max_len);
    if (a.win) L = packed_end(L, a.n_sink, a.n_recent);
  }
  *len = L;
  return id;
}

// value of lane 15 - i of the same 16-lane row (fusable into the consuming VALU op)
__device__ inline float dpp_row_mirror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
}

// Lane swaps of gfx950. v_permlane16_swap(x, y) exchanges the odd 16-lane rows of x
// with the even rows of y (permlane32_swap: the upper half of x with the lower half of
// y); the second operand is an opaque copy (see opaque()).
// value of lane l ^ 16 and of lane l ^ 32
__device__ inline float xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane16_swap(u, opaque(u), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? p[0] : p[1]);
}
__device__ inline float xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, opaque(u), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? p[0] : p[1]);
}
// max / sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ inline float max_over_q(float x) {
  x = fmaxf(x, xor16(x));
  return fmaxf(x, xor32(x));
}
__device__ inline float sum_over_q(float x) {
  x += xor16(x);
  return x + xor32(x);
}
// value of lane l ^ 48 through the LDS crossbar, one instruction per value (lane = this
// lane's index): cheaper than two lane swaps where many values move at once
__device__ inline float lane_xor48(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 48) << 2, __builtin_bit_cast(int, x)));
}

// ---------------------------------------------------------------- query rotation

// One workgroup (1024 threads) per row tile: the tile's query rows in record order, then
// r_g = Pi_g q_g on the VALU: thread (record position i, part p of 8) sums its eighth of
// row i - pos_off[g] of Pi_g against every row of the tile (one round of rotation loads
// per thread, the query pairs broadcast from LDS), the 8 parts add up through lane
// shuffles, and part 0 writes the scaled high and low binary16 halves into the tile's B
// operand. Tiles of 8 rows (RT = 8) put the high parts in columns 0..7 and the low parts
// of rows 7..0 in columns 8..15; tiles of 16 rows (RT = 16, prefill) write two operands,
// high parts then low parts, with row n in column n.
constexpr int kQrotWaves = 16;
// mid() runs once this thread's loads are issued (the decode step's prepare puts a token
// append there, so that both bodies' loads are in flight together); QJL_OK = false leaves the
// sketch rows unloaded (callers that never see a QJL plan).
template <int RT, bool QJL_OK = true, typename Mid>
__device__ __attribute__((always_inline)) inline void qrot_body_with(const AttnArgs& a, int tile, Mid&& mid) {
  constexpr int kParts = RT / 8;       // B operands per tile (1, or 2 for hi and lo)
  constexpr int kTileQB = kParts * kQB;
  __shared__ __align__(16) float qnat[RT][kD];
  __shared__ __align__(16) float qrec[RT][kD];
  __shared__ uint4 qb[kParts * kMaxKB][4][16];
  constexpr int kT = 64 * kQrotWaves;
  const int tid = threadIdx.x;
  int seq, h, tr;
  tile_coords(a, tile, &seq, &h, &tr);
  const DevHead* __restrict__ hp = a.heads + h;
  const GroupLayout GL = load_layout(hp);
  // this thread's output: record position i, its group g, row ii of Pi_g, and its
  // eighth [plo, phi) of the d / 2 column pairs
  const int i = tid >> 3, part = tid & 7;
  const int g = group_of(GL, i);
  const int d = pick(GL.dim, g), po = pick(GL.pos, g), ii = i - po, dp = d >> 1;
  const int plo = (dp * part) >> 3, phi = (dp * (part + 1)) >> 3;
  // one round of loads: the rotation pairs, the tile's query rows (natural order) and
  // the head's record order
  float2 pr[8];
  {
    const float2* row = reinterpret_cast<const float2*>(a.rot + pick(GL.krot, g) + (size_t)ii * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) pr[u] = (plo + u < phi) ? row[plo + u] : make_float2(0.f, 0.f);
  }
  float qv[RT * kD / kT > 0 ? RT * kD / kT : 1];
#pragma unroll
  for (int pp = 0; pp < RT * kD / kT; ++pp) {
    const int r = (tid >> 7) + (kT / kD) * pp, c = tid & (kD - 1);
    int L;
    const int id = tile_row<RT>(a, seq, h, tr, r, 0, &L);
    qv[pp] = id >= 0 ? a.q[(size_t)id * kD + c] : 0.f;
  }
  const int crd = tid < kD ? hp->coord[tid] : 0;
  // QJL plans (decode tiles): this thread's sixteenth of row i of the sketch matrix S
  const bool qjl = RT == 8 && QJL_OK && a.qjl;
  float4 sr[4];
  {
    const float4* row = reinterpret_cast<const float4*>(a.rot + hp->qjl_off + (size_t)i * kD + 16 * part);
#pragma unroll
    for (int u = 0; u < 4; ++u) sr[u] = qjl ? row[u] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  mid();
  __shared__ uint4 qjb[4][4][16];
#pragma unroll
  for (int pp = 0; pp < RT * kD / kT; ++pp) (&qnat[0][0])[tid + kT * pp] = qv[pp];
  for (int e = tid; e < kTileQB; e += kT) (&qb[0][0][0])[e] = make_uint4(0, 0, 0, 0);
  if (qjl && tid < 4 * 4 * 16) (&qjb[0][0][0])[tid] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  if (tid < kD) {
#pragma unroll
    for (int r = 0; r < RT; ++r) qrec[r][tid] = qnat[r][crd];
  }
  __syncthreads();
  __shared__ float wmax[kQrotWaves];
  float acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float2* x = reinterpret_cast<const float2*>(&qrec[r][po]);
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (plo + u < phi) {
        const float2 xx = x[plo + u];
        s = fmaf(pr[u].x, xx.x, s);
        s = fmaf(pr[u].y, xx.y, s);
      }
    }
    acc[r] = s;
  }
  // the sketch's projection (S q)_i of each row, natural coordinate order
  float aq[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float s = 0.f;
    if (qjl) {
      const float4* x = reinterpret_cast<const float4*>(&qnat[r][16 * part]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 xx = x[u];
        s = fmaf(sr[u].x, xx.x, s);
        s = fmaf(sr[u].y, xx.y, s);
        s = fmaf(sr[u].z, xx.z, s);
        s = fmaf(sr[u].w, xx.w, s);
      }
    }
    aq[r] = s;
  }
  // sum the 8 parts (consecutive lanes)
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    acc[r] += __shfl_xor(acc[r], 1);
    acc[r] += __shfl_xor(acc[r], 2);
    acc[r] += __shfl_xor(acc[r], 4);
    aq[r] += __shfl_xor(aq[r], 1);
    aq[r] += __shfl_xor(aq[r], 2);
    aq[r] += __shfl_xor(aq[r], 4);
  }
  // the sketch operand: the key's factor is gamma and its codes decode to c1 sign_j (the
  // rate-1 centroids), so B = (S q)_j qscale sqrt(pi/2) / (128 c1)
  const float sq_scale = qjl ? a.qscale * 1.2533141373155003f / (128.f * a.cb->c[1][1]) : 0.f;
  // Range of the binary16 high parts: if the tile's largest scaled component exceeds
  // 2^14, every operand of the tile is scaled by the power of two 2^-sq that brings it
  // under (exact); the attention kernels multiply the tile's logits by 2^sq.
  float sc = a.qscale / sqrtf((float)d);
  {
    float lm = 0.f;
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) lm = fmaxf(lm, fmaxf(fabsf(acc[r] * sc), fabsf(aq[r] * sq_scale)));
    }
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
    if ((tid & 63) == 0) wmax[tid >> 6] = lm;
    __syncthreads();
    float tm = 0.f;
#pragma unroll
    for (int w = 0; w < kQrotWaves; ++w) tm = fmaxf(tm, wmax[w]);
    int sq = 0;
    if (tm > 16384.f) {  // (NaN or inf inputs keep sq = 0 and propagate)
      int e;
      frexpf(tm / 16384.f, &e);
      sq = e;
    }
    sc = ldexpf(sc, -sq);
    if (tid == 0) a.tile_xs[tile] = ldexpf(1.f, sq);
    if (qjl && part == 0) {  // (RT == 8: columns r high, 15 - r low)
      const float qs = ldexpf(sq_scale, -sq);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float val = aq[r] * qs;
        const _Float16 hi = (_Float16)val;
        const _Float16 lo = (_Float16)(val - (float)hi);
        reinterpret_cast<_Float16*>(&qjb[i >> 5][(i >> 3) & 3][r])[i & 7] = hi;
        reinterpret_cast<_Float16*>(&qjb[i >> 5][(i >> 3) & 3][15 - r])[i & 7] = lo;
      }
    }
  }
  if (part == 0) {
    const int kp = hp->kp_pos[i];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float val = acc[r] * sc;
      const _Float16 hi = (_Float16)val;
      const _Float16 lo = (_Float16)(val - (float)hi);
      if (RT == 8) {
        reinterpret_cast<_Float16*>(&qb[kp >> 5][(kp >> 3) & 3][r])[kp & 7] = hi;
        reinterpret_cast<_Float16*>(&qb[kp >> 5][(kp >> 3) & 3][15 - r])[kp & 7] = lo;
      } else {
        reinterpret_cast<_Float16*>(&qb[kp >> 5][(kp >> 3) & 3][r])[kp & 7] = hi;
        reinterpret_cast<_Float16*>(&qb[kMaxKB + (kp >> 5)][(kp >> 3) & 3][r])[kp & 7] = lo;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < kTileQB; e += kT) a.qb[(size_t)tile * kTileQB + e] = (&qb[0][0][0])[e];
  if (qjl && tid < 4 * 64) a.qjl_qb[(size_t)tile * 256 + tid] = (&qjb[0][0][0])[tid];
}

template <int RT>
__device__ inline void qrot_body(const AttnArgs& a, int tile) {
  qrot_body_with<RT>(a, tile, [] {});
}

template <int RT>
__global__ void __launch_bounds__(64 * kQrotWaves) attn_qrot_kernel(AttnArgs a) { qrot_body<RT>(a, blockIdx.x); }

// Decode step preparation in one launch: workgroups [0, n_app) append the step's
// tokens (with 3 roles: token w / (3 n_kv), KV head (w / 3) % n_kv, role w % 3; with 1:
// token w / n_kv, KV head w % n_kv), the rest rotate the queries of one row tile each;
// the two kinds share no data.
__global__ void __launch_bounds__(1024) decode_prep_kernel(AppendArgs ap, AttnArgs aa, int n_app, int roles) {
  const int w = blockIdx.x;
  if (w < n_app) {
    if (roles == 1) append_token_body(ap, w / ap.n_kv, w % ap.n_kv, 3);
    else append_token_body(ap, w / (3 * ap.n_kv), (w / 3) % ap.n_kv, w % 3);
  }
  else qrot_body<8>(aa, w - n_app);
}

// The same preparation when every token-head has one workgroup and one row tile (one
// row tile per KV head, many token-heads, no QJL sketch): workgroup w = sequence w / n_kv,
// KV head w % n_kv both appends that token and rotates that tile's queries, with the
// rotation's loads issued before the append, so the launch runs in one round of workgroups
// instead of two.
__global__ void __launch_bounds__(1024) decode_prep_pair_kernel(AppendArgs ap, AttnArgs aa) {
  const int w = blockIdx.x;
  qrot_body_with<8, false>(aa, w, [&] { append_token_body(ap, w / ap.n_kv, w % ap.n_kv, 3); });
}

// fp16 window copies: token t / KV head h (one 128-thread workgroup) to its sink slot
// (pos < n_sink) or its recent ring slot pos % n_recent, binary16 round to nearest even.
struct WindowAppendArgs {
  uint16_t* k_sink;
  uint16_t* v_sink;
  uint16_t* k_rec;
  uint16_t* v_rec;
  const float* k;
  const float* v;
  const int32_t* seq_idx;
  const int64_t* pos;
  unsigned long long* overflow;
  int32_t batch, n_kv, n_sink, sink_slots, n_recent;
};

// coordinate c of input row `row` (token x KV head) as binary16 into the sink slot (pos <
// n_sink) or the recent ring slot pos % n_recent of (seq, h)
__device__ inline void window_store(const WindowAppendArgs& w, size_t row, int seq, int h, int64_t pos, int c) {
  const _Float16 kh = (_Float16)w.k[row * kD + c], vh = (_Float16)w.v[row * kD + c];
  const size_t sh = (size_t)seq * w.n_kv + h;
  uint16_t *kd, *vd;
  int slot, slots;
  if (pos < w.n_sink) {
    kd = w.k_sink;
    vd = w.v_sink;
    slot = (int)pos;
    slots = w.sink_slots;
  } else if (w.n_recent > 0) {
    kd = w.k_rec;
    vd = w.v_rec;
    slot = (int)(pos % w.n_recent);
    slots = w.n_recent;
  } else {
    return;
  }
  kd[(sh * slots + slot) * kD + c] = __builtin_bit_cast(uint16_t, kh);
  vd[((sh * (slots / 8) + slot / 8) * kD + c) * 8 + (slot & 7)] = __builtin_bit_cast(uint16_t, vh);
}

__global__ void __launch_bounds__(kD) window_append_kernel(WindowAppendArgs w) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y, c = threadIdx.x;
  const int seq = w.seq_idx[t];
  const int64_t pos = w.pos[t];
  if (seq < 0 || seq >= w.batch || pos < 0) {
    if (c == 0 && h == 0) atomicAdd(w.overflow, 1ull);
    return;
  }
  window_store(w, (size_t)t * w.n_kv + h, seq, h, pos, c);
}

// ---------------------------------------------------------------- partials

constexpr int kKPitch = 17;  // staged key record pitch in words (k_words <= 16): odd, so the
                             // 16 A-rows of one read fall in distinct banks

struct AttnWave {
  uint32_t ktile[kBlk * kKPitch];    // 32 key records
  float knt[kMaxGroups][kBlk];       // group norms, group-major
  float vn[kBlk];
  uint4 vcodes[2][64];               // value codes of the block, 2 v_bits words per lane
};

// Shared block of a partials workgroup whose row tile has RT rows (8: high/low query
// parts share one B operand; 16: separate high and low B operands).
template <int RT>
constexpr int kQ2Copies = RT == 16 ? 8 : 1;
template <int RT>
struct AttnSharedT {
  uint4 oct1[256];                   // byte-indexed decode tables (DevCodebook::oct1, quad2)
  uint2 quad2[256][kQ2Copies<RT>];   // (16-row tiles: each entry 8 times, lane l reads copy
                                     // l mod 8, so that random lookups meet fewer bank conflicts)
  uint32_t lut[kPairTable + 4];      // decode table (DevCodebook::pair)
  uint4 qb[(RT / 8) * kMaxKB][4][16];  // QK B operand(s) per K-block and lane
  int32_t row_id[RT];
  int32_t row_len[RT];
  float om[kWaves][RT];
  float ol[kWaves][RT];
  union alignas(16) {
    AttnWave w[kWaves];              // main loop
    float slot[kWaves][8][kD];       // epilogue: 8 accumulator rows of each wave at a time
  } u;
};
using AttnShared = AttnSharedT<8>;

// 8 codes of rate R (code k at bits [k R, (k + 1) R) of F) -> 8 binary16 centroids: one
// table read of the byte of 1-bit codes, two of the bytes of 2-bit codes, else two
// codes per read of the pair table
template <int R, typename SH>
__device__ inline half8 dequant8(const SH& S, uint32_t F) {
  H8 o;
  if constexpr (R == 1) {
    o.v = S.oct1[F & 0xFFu];
  } else if constexpr (R == 2) {
    constexpr int C = sizeof(S.quad2[0]) / sizeof(uint2);  // copies of an entry
    const int c = (int)(threadIdx.x & (C - 1));
    const uint2 x = S.quad2[F & 0xFFu][c], y = S.quad2[(F >> 8) & 0xFFu][c];
    o.u[0] = x.x;
    o.u[1] = x.y;
    o.u[2] = y.x;
    o.u[3] = y.y;
  } else {
    constexpr int base = ((1 << (2 * R)) - 4) / 3;
    constexpr uint32_t m = (1u << (2 * R)) - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.u[j] = S.lut[base + ((F >> (2 * R * j)) & m)];
  }
  return o.h;
}

template <int VB>
__device__ inline uint32_t vfield(const uint32_t (&vw)[2 * VB], int t) {
  if (VB == 1) return (vw[t >> 2] >> (8 * (t & 3))) & 0xFFu;
  if (VB == 2) return (vw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
  if (VB == 4) return vw[t];
  // VB == 3: 24 bits at bit 24 t
  const int bit = 24 * t, w = bit >> 5, s = bit & 31;
  if (s + 24 <= 32) return vw[w] >> s;
  return __builtin_amdgcn_alignbit(vw[w + 1], vw[w], s);
}

// Per-lane registers of one 32-token block: key code words lane + 64 i (KWL of them,
// enough for k_words <= 2 KWL), group norms 2 lane, 2 lane + 1 of the [32][4] block,
// the value norm of token lane & 31 and the value codes of tokens 8q..8q+7 x
// coordinates 8n..8n+7.
template <int VB, int KWL>
struct BlockData {
  uint32_t kr[KWL];
  float2 kn;
  float vn;
  uint32_t vw[2 * VB];
};

// Raw buffer views of one (sequence, KV head) slice of the cache: reads past the end
// return zero, and every address is a scalar base plus a per-lane constant.
struct SliceRsrc {
  __amdgpu_buffer_rsrc_t kc, kn, vc, vn;
};
constexpr int kRawBufferWord3 = 0x00020000;  // untyped 32-bit buffer (gfx9 descriptor)
constexpr int64_t kMaxCapacity = int64_t(1) << 25;  // tokens: 64 B a token per slice stays < 2 GiB

// (the host keeps every slice under 2 GiB). The inputs are uniform; reading them from
// the first lane keeps the descriptor in scalar registers.
__device__ inline __amdgpu_buffer_rsrc_t slice_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>((uint64_t)hi << 32 | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRawBufferWord3);
}

template <int VB, int KWL>
__device__ inline void load_block(BlockData<VB, KWL>& B, const SliceRsrc& R, int t0, int kw, int lane, int voff_v) {
  const int sk = t0 * kw * 4;
#pragma unroll
  for (int i = 0; i < KWL; ++i)  // (words past the block's records are staged to a pad slot)
    B.kr[i] = __builtin_amdgcn_raw_buffer_load_b32(R.kc, 4 * lane + 256 * i, sk, 0);
  B.kn = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(R.kn, 8 * lane, t0 * (kNS * 4), 0));
  B.vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.vn, 4 * (lane & 31), t0 * 4, 0));
  const int sv = t0 * (4 * VB * 4);  // (t0 / 8) blocks of 32 VB words
  // (vector results are bit-cast whole: element reads of them have been miscompiled)
  if (VB == 1) {
    const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R.vc, voff_v, sv, 0));
    B.vw[0] = x.x; B.vw[1] = x.y;
  } else if (VB == 2) {
    const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R.vc, voff_v, sv, 0));
    B.vw[0] = x.x; B.vw[1] = x.y; B.vw[2] = x.z; B.vw[3] = x.w;
  } else if (VB == 3) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R.vc, voff_v + 8 * i, sv, 0));
      B.vw[2 * i] = x.x; B.vw[2 * i + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R.vc, voff_v + 16 * i, sv, 0));
      B.vw[4 * i] = x.x; B.vw[4 * i + 1] = x.y; B.vw[4 * i + 2] = x.z; B.vw[4 * i + 3] = x.w;
    }
  }
}

__device__ inline uint32_t dpp_row_mirror_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);
}

__device__ inline uint32_t lds_u32(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

// Per-lane and per-K-block constants of the QK (set once per workgroup): for K-block i,
// ko = (byte offset in the shared block of the first staged record word this lane reads
// for its half-0 token) << 5 | (bit shift of its first code in that word); the table
// offset of the block's rate and the offset of its group's norm row.
template <int NKB>
struct QkConst {
  uint32_t ko[NKB];
  int w2[NKB];    // 2 R: bits per table index (uniform)
  int lb[NKB];    // byte offset of the rate's pair table in the shared block (uniform)
  int no[NKB];    // byte offset of the group's norm row within knt (uniform)
};

// One step of a wave's online softmax over one staged 32-token block.
// Stage one block into the wave's shared area: key codes (pitch 17), group norms, value
// norms and value codes. The registers are then free for the next block's loads.
template <int VB, int KWL>
__device__ inline void stage_block(AttnWave& W, const BlockData<VB, KWL>& B, int kw, int lane, const int (&st)[KWL]) {
#pragma unroll
  for (int i = 0; i < KWL; ++i) W.ktile[st[i]] = B.kr[i];
  W.knt[2 * (lane & 1)][lane >> 1] = B.kn.x;
  W.knt[2 * (lane & 1) + 1][lane >> 1] = B.kn.y;
  W.vn[lane & 31] = B.vn;  // (lanes l and l + 32 hold the same norm)
#pragma unroll
  for (int i = 0; i < (2 * VB + 3) / 4; ++i) {
    uint4 x;
    x.x = B.vw[4 * i];
    x.y = 4 * i + 1 < 2 * VB ? B.vw[4 * i + 1] : 0u;
    x.z = 4 * i + 2 < 2 * VB ? B.vw[4 * i + 2] : 0u;
    x.w = 4 * i + 3 < 2 * VB ? B.vw[4 * i + 3] : 0u;
    W.vcodes[i][lane] = x;
  }
}

template <int VB, int NKB>
__device__ inline void attn_block16(const AttnSharedT<16>& S, const AttnWave& W, const AttnArgs& a,
                                    int t0, int lane, int q, int n, int my_len, float xs,
                                    const QkConst<NKB>& C, uint32_t nq_off, uint32_t vn_off,
                                    floatx4 (&oacc)[8], float& m_run, float& l_run) {
  const char* sb = reinterpret_cast<const char*>(&S);
  float lg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = 0.f;
  const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
    const char* rp = sb + (C.ko[i] >> 5);
    const uint32_t* r = reinterpret_cast<const uint32_t*>(rp);
    const uint32_t f0 = __builtin_amdgcn_alignbit(r[1], r[0], C.ko[i]);
    const uint32_t f1 = __builtin_amdgcn_alignbit(r[4 * kKPitch + 1], r[4 * kKPitch], C.ko[i]);
    H8 a0, a1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a0.u[j] = lds_u32(sb, C.lb[i] + (__builtin_amdgcn_ubfe(f0, C.w2[i] * j, C.w2[i]) << 2));
      a1.u[j] = lds_u32(sb, C.lb[i] + (__builtin_amdgcn_ubfe(f1, C.w2[i] * j, C.w2[i]) << 2));
    }
    H8 qh, ql;
    qh.v = S.qb[i][q][n];
    ql.v = S.qb[kMaxKB + i][q][n];
    floatx4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, qh.h, z4, 0, 0, 0);
    floatx4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, qh.h, z4, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, ql.h, d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, ql.h, d1, 0, 0, 0);
    const float4 na = *reinterpret_cast<const float4*>(sb + nq_off + C.no[i]);
    const float4 nb = *reinterpret_cast<const float4*>(sb + nq_off + C.no[i] + 16);
    lg[0] = fmaf(na.x, d0[0], lg[0]);
    lg[1] = fmaf(na.y, d0[1], lg[1]);
    lg[2] = fmaf(na.z, d0[2], lg[2]);
    lg[3] = fmaf(na.w, d0[3], lg[3]);
    lg[4] = fmaf(nb.x, d1[0], lg[4]);
    lg[5] = fmaf(nb.y, d1[1], lg[5]);
    lg[6] = fmaf(nb.z, d1[2], lg[6]);
    lg[7] = fmaf(nb.w, d1[3], lg[7]);
  }
  // ---- online softmax of row n over tokens t0 + 8q + j (logits back in true units: the
  //      tile's operands were scaled by 2^-sq, xs = 2^sq)
  const int tb = t0 + 8 * q;
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = (tb + j >= my_len) ? -INFINITY : lg[j] * xs;
  if (a.logits) {
    const int id = S.row_id[n];
    if (id >= 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tb + j < my_len) a.logits[(size_t)id * a.logits_ld + tb + j] = lg[j] * LN2_F;
    }
  }
  float mblk = lg[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mblk = fmaxf(mblk, lg[j]);
  mblk = max_over_q(mblk);
  const bool grow = mblk > m_run;
  if (__any(grow)) {
    const float m_new = grow ? mblk : m_run;
    const bool rescale = grow && m_run != -INFINITY;
    if (__any(rescale)) {
      const float f = rescale ? exp2f(m_run - m_new) : 1.f;
      l_run *= f;
      // accumulator rows 4q + e live in lanes with n == row: fetch their factors
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fe = __shfl(f, 4 * q + e);
#pragma unroll
        for (int t = 0; t < 8; ++t) oacc[t][e] *= fe;
      }
    }
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
  const float4 va = *reinterpret_cast<const float4*>(sb + vn_off);
  const float4 vb4 = *reinterpret_cast<const float4*>(sb + vn_off + 16);
  const float vn[8] = {va.x, va.y, va.z, va.w, vb4.x, vb4.y, vb4.z, vb4.w};
  float p[8], pv[8], pvm = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = (lg[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lg[j] - m_use);
    pv[j] = (p[j] == 0.f) ? 0.f : p[j] * vn[j];
    pvm = fmaxf(pvm, pv[j]);
  }
  // p * nu_V goes to binary16 high and low parts: a row where it passes 2^14 moves its
  // reference up by the power of two that brings it back (an exact rescale of l, acc
  // and this block's p; every lane takes part in the factor exchange)
  pvm = max_over_q(pvm);
  if (__any(pvm > kPvLimit)) {
    int e = 0;
    if (pvm > kPvLimit) frexpf(pvm / kPvLimit, &e);
    const float f = ldexpf(1.f, -e);
    m_run += (float)e;
    l_run *= f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] *= f;
      pv[j] *= f;
    }
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
      const float fe = __shfl(f, 4 * q + ee);
#pragma unroll
      for (int t = 0; t < 8; ++t) oacc[t][ee] *= fe;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) l_run += p[j];
  H8 ph, pl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto hh = __builtin_amdgcn_cvt_pkrtz(pv[2 * k], pv[2 * k + 1]);
    const auto ll = __builtin_amdgcn_cvt_pkrtz(pv[2 * k] - (float)hh[0], pv[2 * k + 1] - (float)hh[1]);
    ph.u[k] = __builtin_bit_cast(uint32_t, hh);
    pl.u[k] = __builtin_bit_cast(uint32_t, ll);
  }
  // ---- PV over the 8 value tiles, high and low parts of p * nu_V
  uint32_t vw[2 * VB];
#pragma unroll
  for (int i = 0; i < (2 * VB + 3) / 4; ++i) {
    const uint4 x = W.vcodes[i][lane];
    vw[4 * i] = x.x;
    if (4 * i + 1 < 2 * VB) vw[4 * i + 1] = x.y;
    if (4 * i + 2 < 2 * VB) vw[4 * i + 2] = x.z;
    if (4 * i + 3 < 2 * VB) vw[4 * i + 3] = x.w;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const half8 bv = dequant8<VB>(S, vfield<VB>(vw, t));
    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph.h, bv, oacc[t], 0, 0, 0);
    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl.h, bv, oacc[t], 0, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

// One partial (m, l, acc) per row for this split, for rows r0 .. r0 + 7 of the tile: the
// waves' (m, l) and accumulator rows (staged in the shared slots) merged by their
// log-sum-exp weights.
template <int NW = kWaves, typename SH>
__device__ inline void write_partials(const AttnArgs& a, const SH& S, int tid, int r0, int chunk_idx) {
  if (tid < 8 * (kD / 4)) {
    const int r8 = tid >> 5, c4 = tid & 31;
    const int r = r0 + r8;
    const int id = S.row_id[r];
    if (id >= 0) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, S.om[w][r]);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      float l = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float mw = S.om[w][r];
          const float sw = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
          const float4 x = *reinterpret_cast<const float4*>(&S.u.slot[w][r8][4 * c4]);
          acc.x = fmaf(sw, x.x, acc.x);
          acc.y = fmaf(sw, x.y, acc.y);
          acc.z = fmaf(sw, x.z, acc.z);
          acc.w = fmaf(sw, x.w, acc.w);
          l = fmaf(sw, S.ol[w][r], l);
        }
      }
      float* dst = a.partials + ((size_t)id * a.n_chunks + chunk_idx) * kPS;
      *reinterpret_cast<float4*>(dst + 4 + 4 * c4) = acc;
      if (c4 == 0) *reinterpret_cast<float4*>(dst) = make_float4(M, l, 0.f, 0.f);
    }
  }
}

// The fp16 window's split of one 8-row tile (decode with sink and recent buffers), in
// the original basis: QK with A = the binary16 keys (four 32-coordinate K-blocks) and
// B = the queries split into binary16 high and low parts (rows as in the packed
// tiles), the same online softmax, PV with B = the binary16 values, then the waves'
// merge and acc_rot = sqrt(128) Pi_V acc, so that the merge treats it as a packed split.
// Slots that hold no visible position are masked, and their values zeroed before the
// products (unfilled slots may hold anything). Runs in workgroups of the query-rotation
// launch (1024 threads): waves 0..7 do the work, the others only join the barriers.
__device__ inline bool window_slot(const AttnArgs& a, bool sink, int slot, int L, int* pos) {
  if (sink) {
    *pos = slot;
    return slot < a.n_sink && slot < L;
  }
  const int base = L - a.n_recent;  // recent slot r holds the position in [L - W, L) congruent to r
  int d = (slot - base) % a.n_recent;
  if (d < 0) d += a.n_recent;
  *pos = base + d;
  return *pos >= a.n_sink && *pos >= 0;
}

__device__ inline void window_split(const AttnArgs& a, AttnShared& S, int tile) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, n = lane & 15;
  int seq, h, tr;
  tile_coords(a, tile, &seq, &h, &tr);
  const DevHead* __restrict__ hp = a.heads + h;
  const int L = min(max(a.seq_len[seq], 0), a.max_len);
  const size_t sh = (size_t)seq * a.n_kv + h;
  const bool lo = n >= 8;
  const int my_row = lo ? 15 - n : n;
  const int f = tr * 8 + my_row;
  const int qid = f < a.g ? seq * a.n_q + h * a.g + f : -1;
  const bool active = wave < kWaves;
  if (tid < 8) {
    const int fr = tr * 8 + tid;
    S.row_id[tid] = fr < a.g ? seq * a.n_q + h * a.g + fr : -1;
  }
  // B operands (kept in the shared block): column n < 8 the high parts of row n, column
  // n >= 8 the low parts of row 15 - n; lane (q, n) holds coordinates 32 i + 8 q .. + 7
  // of K-block i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    H8 qb;
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (qid >= 0 && wave == 0) {
      const float4* qp = reinterpret_cast<const float4*>(a.q + (size_t)qid * kD + 32 * i + 8 * q);
      x0 = qp[0];
      x1 = qp[1];
    }
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float val = xv[j] * a.qscale;
      const _Float16 hi = (_Float16)val;
      qb.h[j] = lo ? (_Float16)(val - (float)hi) : hi;
    }
    if (wave == 0) S.qb[i][q][n] = qb.v;
  }
  __syncthreads();
  const int nb_sink = a.sink_slots / kBlk, nb = nb_sink + a.n_recent / kBlk;
  const int tau0 = 8 * (n >> 2) + (n & 3);
  floatx4 oacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
  for (int b = wave; active && b < nb; b += kWaves) {
    const bool sink = b < nb_sink;
    const int s0 = sink ? kBlk * b : kBlk * (b - nb_sink);
    const uint16_t* kb = sink ? a.wk_sink + (sh * a.sink_slots + s0) * kD : a.wk_rec + (sh * a.n_recent + s0) * kD;
    const uint16_t* vb = sink ? a.wv_sink + (sh * (a.sink_slots / 8) + s0 / 8) * (kD * 8)
                              : a.wv_rec + (sh * (a.n_recent / 8) + s0 / 8) * (kD * 8);
    // QK over the four K-blocks, both 16-token halves (A-row n: token tau0, tau0 + 4)
    H8 ka[4], kc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i].v = *reinterpret_cast<const uint4*>(kb + (size_t)tau0 * kD + 32 * i + 8 * q);
      kc[i].v = *reinterpret_cast<const uint4*>(kb + (size_t)(tau0 + 4) * kD + 32 * i + 8 * q);
    }
    floatx4 d0 = z4, d1 = z4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      H8 qv;
      qv.v = S.qb[i][q][n];
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i].h, qv.h, d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[i].h, qv.h, d1, 0, 0, 0);
    }
    float lg[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) lg[j] += dpp_row_mirror(lg[j]);
    const int tb = 8 * q + (lo ? 4 : 0);
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int pos;
      const bool ok = window_slot(a, sink, s0 + tb + u, L, &pos);
      x[u] = ok ? (lo ? lg[4 + u] : lg[u]) : -INFINITY;
      if (ok && a.logits) {
        const int id = S.row_id[my_row];
        if (id >= 0) a.logits[(size_t)id * a.logits_ld + pos] = x[u] * LN2_F;
      }
    }
    float mblk = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mblk = fmaxf(mblk, dpp_row_mirror(mblk));
    mblk = max_over_q(mblk);
    const bool grow = mblk > m_run;
    if (__any(grow)) {
      const float m_new = grow ? mblk : m_run;
      const bool rescale = grow && m_run != -INFINITY;
      if (__any(rescale)) {
        const float fac = rescale ? exp2f(m_run - m_new) : 1.f;
        l_run *= fac;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fe = __shfl(fac, 4 * q + e);
#pragma unroll
          for (int t = 0; t < 8; ++t) oacc[t][e] *= fe;
        }
      }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pv[u] = (x[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[u] - m_use);
      l_run += pv[u];
    }
    H8 hv, lv;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto hh = __builtin_amdgcn_cvt_pkrtz(pv[2 * k], pv[2 * k + 1]);
      const auto ll = __builtin_amdgcn_cvt_pkrtz(pv[2 * k] - (float)hh[0], pv[2 * k + 1] - (float)hh[1]);
      hv.u[k] = __builtin_bit_cast(uint32_t, hh);
      lv.u[k] = __builtin_bit_cast(uint32_t, ll);
    }
    H8 pa;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t keep = lo ? lv.u[k] : hv.u[k];
      const uint32_t recv = dpp_row_mirror_u(lo ? hv.u[k] : lv.u[k]);
      pa.u[k] = lo ? recv : keep;
      pa.u[2 + k] = lo ? keep : recv;
    }
    // zero the value halves of slots without a visible position
    uint32_t vm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int pos;
      const bool ok0 = window_slot(a, sink, s0 + 8 * q + 2 * j, L, &pos);
      const bool ok1 = window_slot(a, sink, s0 + 8 * q + 2 * j + 1, L, &pos);
      vm[j] = (ok0 ? 0x0000FFFFu : 0u) | (ok1 ? 0xFFFF0000u : 0u);
    }
    // value operands of the 8 tiles: tokens 8q .. 8q + 7 x coordinate 8n + t
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      H8 bv;
      bv.v = *reinterpret_cast<const uint4*>(vb + ((size_t)q * kD + 8 * n + t) * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) bv.u[j] &= vm[j];
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa.h, bv.h, oacc[t], 0, 0, 0);
    }
  }
  // ---- waves' merge (as in the packed epilogue), then the rotation into the Pi_V basis
  l_run += dpp_row_mirror(l_run);
  l_run = sum_over_q(l_run);
  if (active && q == 0 && n < 8) {
    S.om[wave][n] = m_run;
    S.ol[wave][n] = l_run;
  }
  float vrow[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vrow[t][e] = oacc[t][e] + lane_xor48(oacc[t][3 - e], (int)(threadIdx.x & 63));
  }
  if (active && q < 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float* dst = &S.u.slot[wave][4 * q + e][8 * n];
      *reinterpret_cast<float4*>(dst) = make_float4(vrow[0][e], vrow[1][e], vrow[2][e], vrow[3][e]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(vrow[4][e], vrow[5][e], vrow[6][e], vrow[7][e]);
    }
  }
  // this thread's quarter of a row of Pi_V: output i = tid & 127, inputs 32 qq .. + 31
  const int oi = tid & 127, qq = (tid >> 7) & 3;
  float4 pr[8];
  {
    const float4* pp = reinterpret_cast<const float4*>(a.rot + hp->vrot_off + (size_t)oi * kD + 32 * qq);
#pragma unroll
    for (int u = 0; u < 8; ++u) pr[u] = active ? pp[u] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  float* acc_o = reinterpret_cast<float*>(&S.qb[0][0][0]);  // [8][128] merged rows, then M[8], l[8]
  if (tid < 8 * (kD / 4)) {
    const int r8 = tid >> 5, c4 = tid & 31;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, S.om[w][r8]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = S.om[w][r8];
        const float sw = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        const float4 xx = *reinterpret_cast<const float4*>(&S.u.slot[w][r8][4 * c4]);
        acc.x = fmaf(sw, xx.x, acc.x);
        acc.y = fmaf(sw, xx.y, acc.y);
        acc.z = fmaf(sw, xx.z, acc.z);
        acc.w = fmaf(sw, xx.w, acc.w);
        l = fmaf(sw, S.ol[w][r8], l);
      }
    }
    *reinterpret_cast<float4*>(acc_o + r8 * kD + 4 * c4) = acc;
    if (c4 == 0) {
      acc_o[8 * kD + r8] = M;
      acc_o[8 * kD + 8 + r8] = l;
    }
  }
  __syncthreads();
  float* part = &S.u.slot[0][0][0];  // [4][8][128] quarter sums
#pragma unroll
  for (int r = 0; r < 8 && active; ++r) {
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 xx = *reinterpret_cast<const float4*>(acc_o + r * kD + 32 * qq + 4 * u);
      sum = fmaf(pr[u].x, xx.x, sum);
      sum = fmaf(pr[u].y, xx.y, sum);
      sum = fmaf(pr[u].z, xx.z, sum);
      sum = fmaf(pr[u].w, xx.w, sum);
    }
    part[(qq * 8 + r) * kD + oi] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = tid + kThreads * k;  // 8 rows x 128 outputs
    const int r = e >> 7, i = e & 127;
    const int id = active ? S.row_id[r] : -1;
    if (id >= 0) {
      float* dst = a.partials + ((size_t)(a.sk_G + a.n_tiles + tile) * 8 + r) * kPS;
      const float v = part[(0 * 8 + r) * kD + i] + part[(1 * 8 + r) * kD + i] + part[(2 * 8 + r) * kD + i] +
                      part[(3 * 8 + r) * kD + i];
      dst[4 + i] = v * 11.313708498984761f;  // sqrt(128): the merge divides by it
      if (i == 0) {
        dst[0] = acc_o[8 * kD + r];
        dst[1] = acc_o[8 * kD + 8 + r];
      }
    }
  }
}

// Decode with the fp16 window: workgroups [0, n_tiles) rotate the queries of one row
// tile each, the rest compute the window split of one tile (the two roles share no
// data, and neither reads the packed partials).
__global__ void __launch_bounds__(64 * kQrotWaves) attn_qrot_window_kernel(AttnArgs a, int n_tiles) {
  static_assert(64 * kQrotWaves >= kThreads, "the window split needs 8 waves");
  __shared__ AttnShared S;
  if ((int)blockIdx.x < n_tiles) qrot_body<8>(a, blockIdx.x);
  else window_split(a, S, blockIdx.x - n_tiles);
}

// The prepare launch of a decode step with the fp16 window (one row tile per KV head:
// g <= 8): workgroups [0, n_app) append each sequence's step token (at seq_len - 1) to the
// packed cache, [n_app, n_app + n_tiles) rotate one row tile's queries, the rest first
// write the step token of their tile's sequence and KV head into the fp16 buffers and
// then compute the tile's window split, which reads it.
__global__ void __launch_bounds__(1024) decode_prep_window_kernel(AppendArgs ap, AttnArgs aa, WindowAppendArgs wa,
                                                                   int n_app, int roles, int n_tiles) {
  static_assert(64 * kQrotWaves == 1024, "one block size for the three roles");
  __shared__ AttnShared S;
  const int w = blockIdx.x;
  if (w < n_app) {
    if (roles == 1) append_token_body(ap, w / ap.n_kv, w % ap.n_kv, 3);
    else append_token_body(ap, w / (3 * ap.n_kv), (w / 3) % ap.n_kv, w % 3);
  } else if (w < n_app + n_tiles) {
    qrot_body<8>(aa, w - n_app);
  } else {
    const int tile = w - n_app - n_tiles;
    int seq, h, tr;
    tile_coords(aa, tile, &seq, &h, &tr);
    const int len = aa.seq_len[seq];
    if (len >= 1 && threadIdx.x < kD) window_store(wa, (size_t)seq * wa.n_kv + h, seq, h, (int64_t)len - 1, threadIdx.x);
    __syncthreads();  // (the split below reads the token's slot)
    window_split(aa, S, tile);
  }
}

// Prefill partials: per (row tile of RT = 16 rows, split) online-softmax partials.
// (at most 128 registers: two workgroups per compute unit)
template <int VB, int KWL, int NKB, int RT, bool PAGED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) attn_partials_kernel(AttnArgs a) {
  static_assert(RT == 16, "prefill tiles of 16 rows (decode tiles run attn_decode_kernel)");
  constexpr int kTileQB = (RT / 8) * kQB;
  __shared__ AttnSharedT<RT> S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int q = lane >> 4, n = lane & 15;
  const int chunk_idx = blockIdx.x;
  const int tile = blockIdx.y;
  int seq, h, tr;
  tile_coords(a, tile, &seq, &h, &tr);
  const DevHead* __restrict__ hp = a.heads + h;
  const size_t sh = (size_t)seq * a.n_kv + h;
  const int kw = a.k_words;
  // buffer views of one slice: (sequence, KV head) of a contiguous cache, or (pool page,
  // KV head) of a paged one (an absent page reads as zeros)
  auto slice_views = [&](size_t slice, uint32_t len) {
    SliceRsrc V;
    V.kc = slice_rsrc(a.k_codes + slice * len * kw, len * (uint32_t)kw * 4u);
    V.kn = slice_rsrc(a.k_norms + slice * len * kNS, len * (kNS * 4u));
    V.vc = slice_rsrc(a.v_codes + slice * (len / GTQ_VBLOCK) * (32 * VB), len * (16u * VB));
    V.vn = slice_rsrc(a.v_norms + slice * len, len * 4u);
    return V;
  };
  auto page_views = [&](int pg) {
    const bool ok = pg >= 0 && pg < a.pm.n_pages;
    SliceRsrc V = slice_views((size_t)(ok ? pg : 0) * a.n_kv + h, (uint32_t)a.pm.P);
    if (!ok) V = slice_views(0, 0u);
    return V;
  };
  // the sequence's row of the block table; the page of position t (a vector load, so
  // that it waits with the block loads)
  const __amdgpu_buffer_rsrc_t Rt =
      PAGED ? slice_rsrc(a.pm.table + (size_t)seq * a.pm.tstride, (uint32_t)a.pm.tstride * 4u) : slice_rsrc(a.k_codes, 0u);
  auto page_of = [&](int t) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(Rt, 0, (t >> a.pm.log2P) * 4, 0);
  };
  SliceRsrc R;
  if constexpr (!PAGED) R = slice_views(sh, (uint32_t)a.capacity);
  const int voff_v = 4 * (q * (32 * VB) + n * (2 * VB));
  const int c0 = chunk_idx * a.chunk;
  // ---- one round of independent loads: B operand, decode table, rows, first block
  uint4 qbv[kTileQB / kThreads];
#pragma unroll
  for (int u = 0; u < kTileQB / kThreads; ++u) qbv[u] = a.qb[(size_t)tile * kTileQB + tid + kThreads * u];
  uint32_t lutv[(kPairTable + kThreads - 1) / kThreads];
#pragma unroll
  for (int u = 0; u < (kPairTable + kThreads - 1) / kThreads; ++u) {
    const int e = tid + kThreads * u;
    lutv[u] = e < kPairTable ? a.cb->pair[e] : 0u;
  }
  static_assert(kThreads == 512, "one byte-table entry per thread");
  uint4 tabv;  // threads 0..255: oct1[tid]; 256..511: quad2[tid - 256]
  if (tid < 256) tabv = *reinterpret_cast<const uint4*>(a.cb->oct1[tid]);
  else tabv = make_uint4(a.cb->quad2[tid - 256][0], a.cb->quad2[tid - 256][1], 0u, 0u);
  const int len_ld = a.prefill ? 0 : a.seq_len[seq];
  const float xs = a.tile_xs[tile];
  BlockData<VB, KWL> blk[1];
  int pg_next = 0;
  if constexpr (PAGED) {
    const int t_first = c0 + kBlk * wave;
    load_block<VB, KWL>(blk[0], page_views(__builtin_amdgcn_readfirstlane(page_of(t_first))),
                        t_first & (a.pm.P - 1), kw, lane, voff_v);
    pg_next = page_of(t_first + kBlk * kWaves);
  } else {
    load_block<VB, KWL>(blk[0], R, c0 + kBlk * wave, kw, lane, voff_v);
  }
#pragma unroll
  for (int u = 0; u < kTileQB / kThreads; ++u) (&S.qb[0][0][0])[tid + kThreads * u] = qbv[u];
#pragma unroll
  for (int u = 0; u < (kPairTable + kThreads - 1) / kThreads; ++u) {
    const int e = tid + kThreads * u;
    if (e < kPairTable) S.lut[e] = lutv[u];
  }
  if (tid < 256) {
    S.oct1[tid] = tabv;
  } else {
#pragma unroll
    for (int c = 0; c < kQ2Copies<RT>; ++c) S.quad2[tid - 256][c] = make_uint2(tabv.x, tabv.y);
  }
  if (tid < RT) {
    int L;
    S.row_id[tid] = tile_row<RT>(a, seq, h, tr, tid, len_ld, &L);
    S.row_len[tid] = L;
  }
  __syncthreads();
  int tile_len = 0;
#pragma unroll
  for (int r = 0; r < RT; ++r) tile_len = max(tile_len, S.row_len[r]);
  if (c0 >= tile_len) return;  // no cached token of this tile in this split
  const int c1 = min(c0 + a.chunk, tile_len);
  constexpr int kStep = kBlk * kWaves;

  const int my_len = S.row_len[n];
  AttnWave& W = S.u.w[wave];
  const char* sb = reinterpret_cast<const char*>(&S);
  int st[KWL];  // staging slot of word lane + 64 i: token (lw / kw) at pitch 17; words past
                // the block's 32 records go to the pad column of token 0, whose bits no
                // decoded code uses
#pragma unroll
  for (int i = 0; i < KWL; ++i) {
    const int lw = lane + 64 * i;
    st[i] = lw < kBlk * kw ? (lw / kw) * kKPitch + lw % kw : kKPitch - 1;
  }
  // QK constants: A-row n of the two 16-token halves is token tau0 (+ 4)
  const int tau0 = 8 * (n >> 2) + (n & 3);
  const uint32_t ktile_off = (uint32_t)(reinterpret_cast<const char*>(W.ktile) - sb);
  const uint32_t lut_off = (uint32_t)(reinterpret_cast<const char*>(S.lut) - sb);
  QkConst<NKB> C;
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
    const int rg = hp->kb_rg[i];
    const int rate = rg & 0xFF, grp = rg >> 8;
    const int bit = hp->kb_bit[i] + 8 * q * rate;
    C.ko[i] = ((ktile_off + 4u * (uint32_t)(tau0 * kKPitch + (bit >> 5))) << 5) | (uint32_t)(bit & 31);
    C.w2[i] = 2 * rate;
    C.lb[i] = (int)lut_off + 4 * (((1 << (2 * rate)) - 4) / 3);
    C.no[i] = grp * kBlk * 4;
  }
  const uint32_t nq_off = (uint32_t)(reinterpret_cast<const char*>(&W.knt[0][8 * q]) - sb);
  // value norms: the eight tokens this lane finishes
  const uint32_t vn_off = (uint32_t)(reinterpret_cast<const char*>(&W.vn[8 * q]) - sb);

  floatx4 oacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- main loop: stage the block, start the next block's loads, compute from the stage
  for (int t0 = c0 + kBlk * wave; t0 < c1; t0 += kStep) {
    stage_block<VB, KWL>(W, blk[0], kw, lane, st);
    __builtin_amdgcn_wave_barrier();
    if (t0 + kStep < c1) {
      if constexpr (PAGED) {  // (each 32-token block lies in one page: P is a multiple of 32)
        load_block<VB, KWL>(blk[0], page_views(__builtin_amdgcn_readfirstlane(pg_next)),
                            (t0 + kStep) & (a.pm.P - 1), kw, lane, voff_v);
        pg_next = page_of(t0 + 2 * kStep);
      } else {
        load_block<VB, KWL>(blk[0], R, t0 + kStep, kw, lane, voff_v);
      }
    }
    attn_block16<VB, NKB>(S, W, a, t0, lane, q, n, my_len, xs, C, nq_off, vn_off, oacc, m_run, l_run);
  }

  // ---- epilogue, 16 rows: lane (q, n) holds row n (its l over its own tokens) and the
  //      accumulator rows 4q + e; two rounds of 8 rows through the shared slots
  l_run = sum_over_q(l_run);
  if (q == 0) {
    S.om[wave][n] = m_run;
    S.ol[wave][n] = l_run;
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    __syncthreads();  // hf 0: every wave is done with its stage; hf 1: round 0 was read
    if ((q >> 1) == hf) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* dst = &S.u.slot[wave][4 * (q & 1) + e][8 * n];
        *reinterpret_cast<float4*>(dst) = make_float4(oacc[0][e], oacc[1][e], oacc[2][e], oacc[3][e]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(oacc[4][e], oacc[5][e], oacc[6][e], oacc[7][e]);
      }
    }
    __syncthreads();
    write_partials(a, S, tid, 8 * hf, chunk_idx);
  }
}

// ============================================================================
// Decode partials: tiles of up to 8 query rows of one sequence and KV head (the g query
// heads of the KV head; more than 8 take several tiles).
//
// Work split: the units are the 32-token blocks of every tile's packed range, U in all.
// The launch has G workgroups of 16 waves (one per compute unit by default); workgroup w
// takes units [w U / G, (w + 1) U / G), i.e. the same number of blocks whatever the
// lengths of a ragged batch. Its range crosses tile boundaries: each piece (segment) is
// run by the 16 waves (block b of the segment to wave b mod 16), merged over the waves
// and written as one partial record of its 8 rows at index w + t (unique: a workgroup's
// tiles follow the previous workgroup's last one). The merge finds the segments of a
// tile from the same arithmetic.
//
// Products as in the kernel above (QK: A = decoded key codes of 16 tokens, B = the
// tile's rotated queries as binary16 high/low columns; PV: A = probability times value
// norm in binary16 high/low rows, B = decoded value codes), organised for decode:
//   * K-block slots: the layer's heads order their K-blocks so that the first N1 slots
//     hold rate-1 blocks and the next N4 slots rate-4 blocks in every head of the layer
//     (order_kblocks). A rate-1 slot reads one record byte (eight 1-bit codes) and two
//     entries of the nibble table; a rate-4 slot takes four bytes of its 32-bit field,
//     one pair-table entry each. The products of such a run accumulate in one MFMA chain
//     and meet the group norm once. The remaining slots (rates 2 and 3, blocks past the
//     specialized counts) decode through the pair table of the slot's rate, each scaled
//     by its group norm; slots past the head's count are skipped.
//   * decode tables repeated across the LDS banks (DecTables): random lookups by a wave
//     run at the rate of contiguous reads. They fill most of the 160 KB, hence one
//     workgroup per compute unit.
//   * the query operands and key records / norms are staged in LDS; the value codes go
//     from their loads (issued after the previous block's products) to the products.
//   * softmax against a lazily moved reference: a row's reference m moves only when a
//     logit exceeds it by more than kLazyT (base 2) or p * nu_V would leave the range
//     of the binary16 high parts; that block then takes the exact row maximum, raises
//     m further if a value norm demands it, and rescales. Every other block computes
//     p = 2^(x - m) <= 2^kLazyT with no cross-lane reduction. The partial stores m
//     with l and acc relative to it, which is all the log-sum-exp merge needs.
//   * masking only in blocks that straddle the visible range.
// ============================================================================
constexpr float kLazyT = 10.f;
constexpr int kDecWaves = 16;        // one 1024-thread workgroup per compute unit
constexpr int kDecThreads = 64 * kDecWaves;

struct DecWave {
  uint32_t ktile[kBlk * kKPitch];    // 32 key records, pitch 17 words
  float knt[kMaxGroups + 1][kBlk];   // key group norms, group-major, then the QJL gamma
  float vn[kBlk];                    // value norms
};
// Decode tables in LDS, each entry repeated so that a wave's random lookups fall in
// distinct banks: entry e of a table kept R times sits at (e R + r) x its size and lane
// l reads copy r = l mod R. The copy counts are the smallest a random wave-wide read of
// that width needs to run at the rate of a contiguous one on gfx950 (b64: 32; the b32
// pair tables of rates 3 and 4 keep 32 and 16 for space). Byte offsets are fixed (the
// lookups put them in the instruction's offset field).
constexpr uint32_t kDecT1 = 4096, kDecP3 = 8192, kDecP4 = 16384, kDecQ2 = 32768;
struct DecTables {
  uint32_t lut[1024];                // all pair tables once (DevCodebook::pair); the rate-1
                                     // and rate-2 ones (4 and 16 entries) read conflict-free
  uint2 t1[16][32];                  // 4 rate-1 centroids of each nibble, 32 copies
  uint32_t p3[64][32];               // rate-3 pairs, 32 copies
  uint32_t p4[256][16];              // rate-4 pairs, 16 copies
  uint2 q2[256][32];                 // 4 rate-2 centroids of each byte, 32 copies
};
static_assert(offsetof(DecTables, t1) == kDecT1 && offsetof(DecTables, p3) == kDecP3 &&
                  offsetof(DecTables, p4) == kDecP4 && offsetof(DecTables, q2) == kDecQ2,
              "decode table offsets");
struct DecShared {
  union alignas(16) {
    DecTables t;
  } u;
  DecWave w[kDecWaves];              // main loop (reads of partial K-blocks may run a few words
                                     // past a wave's records: still inside S); between a
                                     // segment's loop and its partial, eight merge slots
  long long sk_u0, sk_u1, sk_P;      // this workgroup's next unit, its end, the units before sk_b
  long long sk_U;                    // all units of the batch
  int32_t sk_b;                      // the sequence of the next unit (or an earlier, empty one)
  int32_t sk_tile;                   // the current segment's row tile
  uint4 qb[kMaxKB - 1][4][16];       // query operands of the K-block slots
  uint4 qjlb[4][4][16];              // QJL plans: the residual sketch's operands
  int32_t row_id[8];
  int32_t row_len[8];
  alignas(16) float om[kDecWaves][8];  // (rows read as float4)
  float ol[kDecWaves][8];
};
static_assert(offsetof(DecShared, u) == 0, "tables at the start of the shared block");

// Lane base offsets of the replicated tables: copy lane mod 32 of an 8-byte table
// (t1, q2), lane mod 32 and lane mod 16 of a 4-byte one (p3, p4)
struct DecLanes {
  uint32_t l8, l4_32, l4_16;
};

__device__ inline uint2 lds_u64(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint2*>(base + off);
}

// the 8 binary16 centroids of the 8 codes of rate R in F (code k at bits R k) from the
// replicated tables: nibbles through t1 (R = 1), bytes through q2 (R = 2), code pairs
// through p3 / p4 (R = 3, 4)
template <int R>
__device__ inline half8 dec_dequant8(const char* sb, const DecLanes& L, uint32_t F) {
  H8 o;
  if constexpr (R == 1) {
    const uint2 x = lds_u64(sb, kDecT1 + (((F << 8) & 0xF00u) | L.l8));
    const uint2 y = lds_u64(sb, kDecT1 + (((F << 4) & 0xF00u) | L.l8));
    o.u[0] = x.x; o.u[1] = x.y; o.u[2] = y.x; o.u[3] = y.y;
  } else if constexpr (R == 2) {
    const uint2 x = lds_u64(sb, kDecQ2 + (((F << 8) & 0xFF00u) | L.l8));
    const uint2 y = lds_u64(sb, kDecQ2 + ((F & 0xFF00u) | L.l8));
    o.u[0] = x.x; o.u[1] = x.y; o.u[2] = y.x; o.u[3] = y.y;
  } else if constexpr (R == 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o.u[j] = lds_u32(sb, kDecP3 + ((__builtin_amdgcn_ubfe(F, 6 * j, 6) << 7) | L.l4_32));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o.u[j] = lds_u32(sb, kDecP4 + ((__builtin_amdgcn_ubfe(F, 8 * j, 8) << 6) | L.l4_16));
  }
  return o.h;
}

template <int VB, int KWL>
struct DecBlock {
  uint32_t kr[KWL];
  float2 kn;
  float vn;
  uint32_t vw[2 * VB];
};

// Loads of one 32-token block (raw buffer views: reads past the slice return 0). Key
// words: with W = 2 KWL words per record row, lane l takes word l mod W of tokens
// l / W + (64 / W) i (kvo = its byte offset in the block's records; lanes with
// l mod W >= kw read the next record's first words, which land in the pad of their row).
// Key norms 2 lane, 2 lane + 1 of the [32][4] block and the value norm of token lane & 31
// (dec_load_k); this lane's value words, tokens 8q..8q+7 x coordinates 8n..8n+7
// (dec_load_v: issued once the products of the previous block have read them).
template <int VB, int KWL>
__device__ inline void dec_load_k(DecBlock<VB, KWL>& B, const SliceRsrc& R, int t0, int kw, int lane, int kvo) {
  const int sk = t0 * kw * 4;
  constexpr int kTok = 64 / (2 * KWL);  // tokens per load instruction
#pragma unroll
  for (int i = 0; i < KWL; ++i) B.kr[i] = __builtin_amdgcn_raw_buffer_load_b32(R.kc, kvo, sk + i * kTok * kw * 4, 0);
  B.kn = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(R.kn, 8 * lane, t0 * (kNS * 4), 0));
  B.vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.vn, 4 * (lane & 31), t0 * 4, 0));
}
template <int VB, int KWL>
__device__ inline void dec_load_v(DecBlock<VB, KWL>& B, const SliceRsrc& R, int t0, int voff_v) {
  const int sv = t0 * (4 * VB * 4);
  if (VB == 1) {
    const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R.vc, voff_v, sv, 0));
    B.vw[0] = x.x; B.vw[1] = x.y;
  } else if (VB == 2) {
    const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R.vc, voff_v, sv, 0));
    B.vw[0] = x.x; B.vw[1] = x.y; B.vw[2] = x.z; B.vw[3] = x.w;
  } else if (VB == 3) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R.vc, voff_v + 8 * i, sv, 0));
      B.vw[2 * i] = x.x; B.vw[2 * i + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R.vc, voff_v + 16 * i, sv, 0));
      B.vw[4 * i] = x.x; B.vw[4 * i + 1] = x.y; B.vw[4 * i + 2] = x.z; B.vw[4 * i + 3] = x.w;
    }
  }
}

// max over the lanes of a row: lanes n, 15 - n (row mirror) and q = 0..3
__device__ inline float row_max(float x) {
  x = fmaxf(x, dpp_row_mirror(x));
  return max_over_q(x);
}

template <int VB, int KWL, int N1, int N4, bool PAGED, bool QJL>
__global__ void __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) attn_decode_kernel(AttnArgs a) {
  constexpr int NS = kMaxKB - 1;  // K-block slots (a head has at most 7)
  __shared__ DecShared S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, n = lane & 15;
  const int kw = a.k_words;
  const int G = gridDim.x, wg = blockIdx.x;
  const int tps = a.n_kv * a.tiles_per_kv;  // row tiles per sequence
  int seq = 0, h = 0;                        // of the current segment (the views read them)
  constexpr bool paged = PAGED;
  using KArgs = const __attribute__((address_space(4))) AttnArgs;
  KArgs* const ka0 = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  auto slice_views_of = [&](const AttnArgs& A, size_t slice, uint32_t len) {
    SliceRsrc V;
    V.kc = slice_rsrc(A.k_codes + slice * len * kw, len * (uint32_t)kw * 4u);
    V.kn = slice_rsrc(A.k_norms + slice * len * kNS, len * (kNS * 4u));
    V.vc = slice_rsrc(A.v_codes + slice * (len / GTQ_VBLOCK) * (32 * VB), len * (16u * VB));
    V.vn = slice_rsrc(A.v_norms + slice * len, len * 4u);
    return V;
  };
  auto slice_views = [&](size_t slice, uint32_t len) {
    SliceRsrc V;
    V.kc = slice_rsrc(a.k_codes + slice * len * kw, len * (uint32_t)kw * 4u);
    V.kn = slice_rsrc(a.k_norms + slice * len * kNS, len * (kNS * 4u));
    V.vc = slice_rsrc(a.v_codes + slice * (len / GTQ_VBLOCK) * (32 * VB), len * (16u * VB));
    V.vn = slice_rsrc(a.v_norms + slice * len, len * 4u);
    return V;
  };
  auto page_views = [&](int pg) {
    const bool ok = pg >= 0 && pg < a.pm.n_pages;
    SliceRsrc V = slice_views((size_t)(ok ? pg : 0) * a.n_kv + h, (uint32_t)a.pm.P);
    if (!ok) V = slice_views(0, 0u);
    return V;
  };
  auto page_of = [&](int t) {
    const __amdgpu_buffer_rsrc_t Rt = slice_rsrc(a.pm.table + (size_t)seq * a.pm.tstride, (uint32_t)a.pm.tstride * 4u);
    return (int)__builtin_amdgcn_raw_buffer_load_b32(Rt, 0, (t >> a.pm.log2P) * 4, 0);
  };
  constexpr int kRowW = 2 * KWL;  // record words a lane row covers (>= kw)
  // ---- the replicated tables (entries through registers), and this workgroup's units
  const DevCodebook* __restrict__ cb = a.cb;
  static_assert(kPairTable <= kDecThreads && 16 * 32 <= kDecThreads, "one entry per thread");
  constexpr int kU3 = 64 * 64 / kDecThreads, kU2 = 256 * 32 / kDecThreads;
  const uint32_t lutv = tid < kPairTable ? cb->pair[tid] : 0u;
  const uint2 t1v = *reinterpret_cast<const uint2*>(cb->oct1[(tid >> 5) & 15]);
  uint32_t p3v[kU3], p4v[kU3];
  uint2 q2v[kU2];
#pragma unroll
  for (int u = 0; u < kU3; ++u) {
    const int e = tid + kDecThreads * u;
    p3v[u] = cb->pair[20 + (e >> 5)];  // (the first kU3 / 2 rounds; the rest unused)
    p4v[u] = cb->pair[84 + (e >> 4)];
  }
#pragma unroll
  for (int u = 0; u < kU2; ++u) q2v[u] = *reinterpret_cast<const uint2*>(cb->quad2[(tid + kDecThreads * u) >> 5]);
  if (wave == 0) {
    // U = all units; this workgroup's range [u0, u1); the first sequence b with units at
    // or past u0 and P = the units before it
    long long U = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      const int b = b0 + lane;
      long long x = b < a.batch ? (long long)tps * seq_blocks(a.seq_len, b, a.max_len, a.win, a.n_sink, a.n_recent) : 0;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
      U += x;
    }
    const long long u0 = (long long)wg * U / G, u1 = (long long)(wg + 1) * U / G;
    long long P = 0, Ps = 0;
    int bs = -1;
    for (int b0 = 0; b0 < a.batch && bs < 0; b0 += 64) {
      const int b = b0 + lane;
      const long long x =
          b < a.batch ? (long long)tps * seq_blocks(a.seq_len, b, a.max_len, a.win, a.n_sink, a.n_recent) : 0;
      long long incl = x;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const long long y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      incl += P;
      const unsigned long long hit = __ballot(b < a.batch && incl > u0);
      if (hit) {
        const int f = __ffsll((long long)hit) - 1;
        bs = b0 + f;
        Ps = __shfl(incl - x, f);
      }
      P = __shfl(incl, 63);
    }
    if (lane == 0) {
      S.sk_u0 = u0;
      S.sk_u1 = u1;
      S.sk_P = Ps;
      S.sk_b = bs;
      S.sk_U = U;
    }
  }
  if (tid < kPairTable) S.u.t.lut[tid] = lutv;
  if (tid < 16 * 32) S.u.t.t1[tid >> 5][tid & 31] = t1v;
#pragma unroll
  for (int u = 0; u < kU3; ++u) {
    const int e = tid + kDecThreads * u;
    if (e < 64 * 32) S.u.t.p3[e >> 5][e & 31] = p3v[u];
    S.u.t.p4[e >> 4][e & 15] = p4v[u];
  }
#pragma unroll
  for (int u = 0; u < kU2; ++u) {
    const int e = tid + kDecThreads * u;
    S.u.t.q2[e >> 5][e & 31] = q2v[u];
  }
  __syncthreads();
  constexpr int kStep = kBlk * kDecWaves;
  const char* sb = reinterpret_cast<const char*>(&S);
  const uint8_t* sb8 = reinterpret_cast<const uint8_t*>(sb);
  const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
  float* const slots = reinterpret_cast<float*>(&S.w[0]);  // [8][8][kD] in the wave areas (epilogue)
  DecWave& W = S.w[wave];

  // ---- the segments: blocks [bb, be) of row tile `tile`, one partial each. The position
  //      (next unit, sequence, units before it) lives in the shared block between segments.
  auto rfl64 = [](long long x) {
    const int lo32 = __builtin_amdgcn_readfirstlane((int)(x & 0xFFFFFFFFll));
    const int hi32 = __builtin_amdgcn_readfirstlane((int)(x >> 32));
    return (long long)(((unsigned long long)(unsigned)hi32 << 32) | (unsigned)lo32);
  };
  for (;;) {
    // the arguments the segment set-up reads are loaded again here rather than held in
    // registers across the main loop
    KArgs* kap = ka0;
    asm volatile("" : "+s"(kap));
    const AttnArgs& A = *(const AttnArgs*)kap;
    // the lane's constants, from an opaque copy of the thread index: derived again for each
    // segment rather than held in registers across the segment loop
    int tid_v = threadIdx.x;
    asm volatile("" : "+v"(tid_v));
    const int tid = tid_v, lane = tid & 63, q = lane >> 4, n = lane & 15;
    const int voff_v = 4 * (q * (32 * VB) + n * (2 * VB));
    const int kvo = 4 * ((lane / kRowW) * kw + lane % kRowW);
    const bool lo = n >= 8;
    const int lo_vis = A.win ? A.n_sink : 0;  // sink positions read the fp16 buffers
    const int my_row = lo ? 15 - n : n;
    const int kst = (lane / kRowW) * kKPitch + lane % kRowW;  // LDS word of the lane's first key word
    // A-row n of the two 16-token halves: token tau0 and tau0 + 4
    const int tau0 = 8 * (n >> 2) + (n & 3);
    const uint32_t ktile_off = (uint32_t)(reinterpret_cast<const char*>(W.ktile) - sb);
    const uint32_t row0 = ktile_off + 4u * (uint32_t)(tau0 * kKPitch);  // byte offset of token tau0's record
    constexpr uint32_t kHalf = 4u * 4u * kKPitch;                       // token tau0 + 4
    DecLanes DL;
    DL.l8 = (uint32_t)(lane & 31) << 3;
    DL.l4_32 = (uint32_t)(lane & 31) << 2;
    DL.l4_16 = (uint32_t)(lane & 15) << 2;
    // this lane's key norms: knt[g][8q .. 8q + 7]
    const uint32_t nq_off = (uint32_t)(reinterpret_cast<const char*>(&W.knt[0][8 * q]) - sb);
    auto knorm4 = [&](int g, int hf) { return *reinterpret_cast<const float4*>(sb + nq_off + g * (kBlk * 4) + 16 * hf); };
    long long u = rfl64(S.sk_u0);
    const long long u_end = rfl64(S.sk_u1);
    if (u >= u_end) break;
    long long Pb = rfl64(S.sk_P);
    int b = __builtin_amdgcn_readfirstlane(S.sk_b);
    int nb = seq_blocks(A.seq_len, b, A.max_len, A.win, A.n_sink, A.n_recent);
    while (nb == 0) nb = seq_blocks(A.seq_len, ++b, A.max_len, A.win, A.n_sink, A.n_recent);  // (no units)
    const int tis = (int)(u - Pb) / nb;  // (the units of one sequence fit in 31 bits)
    const int tile = b * tps + tis;
    const long long Ut = Pb + (long long)tis * nb;
    const int bb = (int)(u - Ut);
    const int be = (int)min((long long)nb, u_end - Ut);
    u = Ut + be;
    if (be == nb && tis == tps - 1) {
      Pb += (long long)tps * nb;
      ++b;
    }
    int tr;
    tile_coords(A, tile, &seq, &h, &tr);
    const DevHead* __restrict__ hp = A.heads + h;
    SliceRsrc R;
    if constexpr (!PAGED) R = slice_views_of(A, (size_t)seq * A.n_kv + h, (uint32_t)A.capacity);
    const int c0 = bb * kBlk;
    // one round of independent loads: query operands (to LDS), rows, the first block
    static_assert(NS * 64 <= kDecThreads, "one query operand per thread");
    const uint4 qg = tid < NS * 64 ? A.qb[(size_t)tile * kQB + tid] : make_uint4(0, 0, 0, 0);
    const uint4 qjg = (QJL && tid < 4 * 64) ? A.qjl_qb[(size_t)tile * 256 + tid] : make_uint4(0, 0, 0, 0);
    const int len_ld = A.seq_len[seq];
    const float xs = A.tile_xs[tile];
    DecBlock<VB, KWL> blk;
    int pg_next = 0;
    {
      const int t_first = c0 + kBlk * wave;
      if constexpr (PAGED) {
        const SliceRsrc R0 = page_views(__builtin_amdgcn_readfirstlane(page_of(t_first)));
        dec_load_k<VB, KWL>(blk, R0, t_first & (A.pm.P - 1), kw, lane, kvo);
        dec_load_v<VB, KWL>(blk, R0, t_first & (A.pm.P - 1), voff_v);
        pg_next = page_of(t_first + kBlk * kDecWaves);
      } else {
        dec_load_k<VB, KWL>(blk, R, t_first, kw, lane, kvo);
        dec_load_v<VB, KWL>(blk, R, t_first, voff_v);
      }
    }
    if (tid < NS * 64) (&S.qb[0][0][0])[tid] = qg;
    if (QJL && tid < 4 * 64) (&S.qjlb[0][0][0])[tid] = qjg;
    if (tid < 8) {
      int L;
      S.row_id[tid] = tile_row<8>(A, seq, h, tr, tid, len_ld, &L);
      S.row_len[tid] = L;
    }
    __syncthreads();  // (every thread has read the position)
    if (tid == 0) {
      S.sk_u0 = u;
      S.sk_P = Pb;
      S.sk_b = b;
      S.sk_tile = tile;
      if (bb == 0) {  // this workgroup runs the tile's first block: the merge's pointers
        const long long Ua = S.sk_U;
        const int w1 = sk_owner(Ut + nb - 1, G, Ua);
        A.tile_info[tile] = make_int4(wg, w1 - wg + 1, (int)(Ua & 0xFFFFFFFFll), (int)(Ua >> 32));
      }
    }
    // every present row of a decode tile has the sequence's length (c0 lies inside it)
    int tile_len = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) tile_len = max(tile_len, S.row_len[r]);
    const int c1 = min(be * kBlk, tile_len);
  const int nkb = hp->nkb;
  const int gl = hp->n_groups - 1;
  // rate-4 slots: the lane's field starts at word (bit >> 5) + q, shift bit & 31 (uniform)
  uint32_t a4[N4 > 0 ? N4 : 1];
  int sh4[N4 > 0 ? N4 : 1];
#pragma unroll
  for (int j = 0; j < N4; ++j) {
    const int bit = hp->kb_bit[N1 + j];
    a4[j] = row0 + 4u * (uint32_t)((bit >> 5) + q);
    sh4[j] = bit & 31;
  }
  // other slots: per-lane LDS address << 5 | shift of the first code; one uniform word
  // with the index width 2R (bits 0..3), the group (bits 4..5), the copy stride shift
  // (bits 6..9: 2 for the single pair tables of rates 1 and 2, 7 for p3, 6 for p4) and
  // the table's byte offset (bits 12..)
  constexpr int NG = NS - N1 - N4;
  uint32_t gko[NG > 0 ? NG : 1];
  uint32_t gpk[NG > 0 ? NG : 1];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int rg = hp->kb_rg[N1 + N4 + i];
    const int rate = rg & 0xFF;
    const int bit = hp->kb_bit[N1 + N4 + i] + 8 * q * rate;
    gko[i] = ((row0 + 4u * (uint32_t)(bit >> 5)) << 5) | (uint32_t)(bit & 31);
    const uint32_t tb = rate == 3 ? kDecP3 : rate == 4 ? kDecP4 : 4u * (uint32_t)(((1 << (2 * rate)) - 4) / 3);
    const uint32_t ts = rate == 3 ? 7u : rate == 4 ? 6u : 2u;
    gpk[i] = (uint32_t)(2 * rate) | (uint32_t)(rg >> 8) << 4 | ts << 6 | tb << 12;
  }

  floatx4 oacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f, thr = -INFINITY;

  for (int t0 = c0 + kBlk * wave; t0 < c1; t0 += kStep) {
    // ---- stage the key records and key norms; the value words and norms stay in registers
#pragma unroll
    for (int i = 0; i < KWL; ++i) W.ktile[kst + i * (64 / kRowW) * kKPitch] = blk.kr[i];
    if (QJL && lane % kRowW == a.mse_words + 4) {  // the QJL gamma (record word mse + 4)
#pragma unroll
      for (int i = 0; i < KWL; ++i) W.knt[kMaxGroups][lane / kRowW + i * (64 / kRowW)] = __builtin_bit_cast(float, blk.kr[i]);
    }
    W.knt[2 * (lane & 1)][lane >> 1] = blk.kn.x;
    W.knt[2 * (lane & 1) + 1][lane >> 1] = blk.kn.y;
    W.vn[lane & 31] = blk.vn;  // (lanes l and l + 32 hold the same norm)
    __builtin_amdgcn_wave_barrier();
    // the next block: key part now, value words after this block's products
    // (a 32-token block lies in one page: P is a multiple of 32)
    const bool more = t0 + kStep < c1;
    const int t_next = PAGED ? (t0 + kStep) & (a.pm.P - 1) : t0 + kStep;
    if (more) {
      if constexpr (PAGED) dec_load_k<VB, KWL>(blk, page_views(__builtin_amdgcn_readfirstlane(pg_next)), t_next, kw, lane, kvo);
      else dec_load_k<VB, KWL>(blk, R, t_next, kw, lane, kvo);
    }
    // ---- QK: lg[4 hf + e] = logit (high or low column part) of token 8q + 4 hf + e
    float lg[8];
    if constexpr (N1 > 0) {
      floatx4 d0 = z4, d1 = z4;
#pragma unroll
      for (int i = 0; i < N1; ++i) {
        H8 a0, a1;
        a0.h = dec_dequant8<1>(sb, DL, sb8[row0 + 4 * i + q]);
        a1.h = dec_dequant8<1>(sb, DL, sb8[row0 + kHalf + 4 * i + q]);
        H8 bq;
        bq.v = S.qb[i][q][n];
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, bq.h, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, bq.h, d1, 0, 0, 0);
      }
      const float4 na = knorm4(0, 0), nb = knorm4(0, 1);
      lg[0] = na.x * d0[0]; lg[1] = na.y * d0[1]; lg[2] = na.z * d0[2]; lg[3] = na.w * d0[3];
      lg[4] = nb.x * d1[0]; lg[5] = nb.y * d1[1]; lg[6] = nb.z * d1[2]; lg[7] = nb.w * d1[3];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) lg[j] = 0.f;
    }
    if constexpr (N4 > 0) {
      floatx4 d0 = z4, d1 = z4;
#pragma unroll
      for (int j = 0; j < N4; ++j) {
        const uint32_t* r = reinterpret_cast<const uint32_t*>(sb + a4[j]);
        const uint32_t f0 = __builtin_amdgcn_alignbit(r[1], r[0], sh4[j]);
        const uint32_t f1 = __builtin_amdgcn_alignbit(r[4 * kKPitch + 1], r[4 * kKPitch], sh4[j]);
        H8 a0, a1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a0.u[k] = lds_u32(sb, kDecP4 + ((__builtin_amdgcn_ubfe(f0, 8 * k, 8) << 6) | DL.l4_16));
          a1.u[k] = lds_u32(sb, kDecP4 + ((__builtin_amdgcn_ubfe(f1, 8 * k, 8) << 6) | DL.l4_16));
        }
        H8 bq;
        bq.v = S.qb[N1 + j][q][n];
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, bq.h, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, bq.h, d1, 0, 0, 0);
      }
      const float4 na = knorm4(gl, 0), nb = knorm4(gl, 1);
      lg[0] = fmaf(na.x, d0[0], lg[0]); lg[1] = fmaf(na.y, d0[1], lg[1]);
      lg[2] = fmaf(na.z, d0[2], lg[2]); lg[3] = fmaf(na.w, d0[3], lg[3]);
      lg[4] = fmaf(nb.x, d1[0], lg[4]); lg[5] = fmaf(nb.y, d1[1], lg[5]);
      lg[6] = fmaf(nb.z, d1[2], lg[6]); lg[7] = fmaf(nb.w, d1[3], lg[7]);
    }
    if constexpr (QJL) {
      // the residual sketch: four 32-bit slots after the MSE words, decoded like rate-1
      // codes (centroids c1 sign_j) against B = S q scaled, times gamma
      floatx4 d0 = z4, d1 = z4;
      const uint32_t sk0 = row0 + 4u * (uint32_t)a.mse_words;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        H8 a0, a1, bq;
        a0.h = dec_dequant8<1>(sb, DL, sb8[sk0 + 4 * i + q]);
        a1.h = dec_dequant8<1>(sb, DL, sb8[sk0 + kHalf + 4 * i + q]);
        bq.v = S.qjlb[i][q][n];
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, bq.h, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, bq.h, d1, 0, 0, 0);
      }
      const float4 na = knorm4(kMaxGroups, 0), nb = knorm4(kMaxGroups, 1);
      lg[0] = fmaf(na.x, d0[0], lg[0]); lg[1] = fmaf(na.y, d0[1], lg[1]);
      lg[2] = fmaf(na.z, d0[2], lg[2]); lg[3] = fmaf(na.w, d0[3], lg[3]);
      lg[4] = fmaf(nb.x, d1[0], lg[4]); lg[5] = fmaf(nb.y, d1[1], lg[5]);
      lg[6] = fmaf(nb.z, d1[2], lg[6]); lg[7] = fmaf(nb.w, d1[3], lg[7]);
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (N1 + N4 + i < nkb) {
        const uint32_t* r = reinterpret_cast<const uint32_t*>(sb + (gko[i] >> 5));
        const uint32_t f0 = __builtin_amdgcn_alignbit(r[1], r[0], gko[i]);
        const uint32_t f1 = __builtin_amdgcn_alignbit(r[4 * kKPitch + 1], r[4 * kKPitch], gko[i]);
        const uint32_t w2 = gpk[i] & 15u, ts = (gpk[i] >> 6) & 15u;
        const uint32_t lb = (gpk[i] >> 12) + (ts == 7u ? DL.l4_32 : ts == 6u ? DL.l4_16 : 0u);
        H8 a0, a1, bq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a0.u[j] = lds_u32(sb, lb + (__builtin_amdgcn_ubfe(f0, w2 * j, w2) << ts));
          a1.u[j] = lds_u32(sb, lb + (__builtin_amdgcn_ubfe(f1, w2 * j, w2) << ts));
        }
        bq.v = S.qb[N1 + N4 + i][q][n];
        const floatx4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.h, bq.h, z4, 0, 0, 0);
        const floatx4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.h, bq.h, z4, 0, 0, 0);
        const int grp = (int)((gpk[i] >> 4) & 3u);
        const float4 na = knorm4(grp, 0), nb = knorm4(grp, 1);
        lg[0] = fmaf(na.x, d0[0], lg[0]); lg[1] = fmaf(na.y, d0[1], lg[1]);
        lg[2] = fmaf(na.z, d0[2], lg[2]); lg[3] = fmaf(na.w, d0[3], lg[3]);
        lg[4] = fmaf(nb.x, d1[0], lg[4]); lg[5] = fmaf(nb.y, d1[1], lg[5]);
        lg[6] = fmaf(nb.z, d1[2], lg[6]); lg[7] = fmaf(nb.w, d1[3], lg[7]);
      }
    }
    // ---- whole logits (high + low columns); this lane finishes tokens 8q + 4 lo + u of
    //      row my_row, in units of 2^-sq (xs = 2^sq)
#pragma unroll
    for (int j = 0; j < 8; ++j) lg[j] += dpp_row_mirror(lg[j]);
    const int tb = t0 + 8 * q + (lo ? 4 : 0);
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = lo ? lg[4 + u] : lg[u];
    const bool edge = (t0 + kBlk > c1) || (t0 < lo_vis);  // uniform
    if (edge) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tb + u >= c1 || tb + u < lo_vis) x[u] = -INFINITY;
    }
    if (a.logits) {
      const int id = S.row_id[my_row];
      if (id >= 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (tb + u < c1 && tb + u >= lo_vis) a.logits[(size_t)id * a.logits_ld + tb + u] = x[u] * xs * LN2_F;
      }
    }
    // ---- softmax against the lazily moved reference m_ref (base 2)
    const float4 vn4 = *reinterpret_cast<const float4*>(&W.vn[8 * q + (lo ? 4 : 0)]);
    const float vn[4] = {vn4.x, vn4.y, vn4.z, vn4.w};
    float p[4], pv[4];
    {
      const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
      float xm = -INFINITY, pm = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xm = fmaxf(xm, x[u]);
        p[u] = __builtin_amdgcn_exp2f(fmaf(x[u], xs, -mu));
        pv[u] = p[u] * vn[u];
        pm = fmaxf(pm, pv[u]);
      }
      if (edge) {  // masked tokens contribute nothing, whatever their value norm holds
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = (x[u] == -INFINITY) ? 0.f : pv[u];
      }
      if (__any(xm > thr || !(pm <= kPvLimit))) {
        // exact row maximum of this block; the reference moves to the larger of it and
        // the old one, then further by the power of two that keeps p * nu_V <= 2^14
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) mb = fmaxf(mb, x[u] * xs);
        mb = row_max(mb);
        float m_new = fmaxf(m_ref, mb);
        const float mu2 = (m_new == -INFINITY) ? 0.f : m_new;
        float pvm = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = __builtin_amdgcn_exp2f(fmaf(x[u], xs, -mu2));
          pv[u] = (x[u] == -INFINITY) ? 0.f : p[u] * vn[u];
          pvm = fmaxf(pvm, pv[u]);
        }
        pvm = row_max(pvm);
        if (pvm > kPvLimit && m_new != -INFINITY) {  // (a NaN value norm stays NaN)
          int e;
          frexpf(pvm / kPvLimit, &e);
          m_new += (float)e;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            p[u] = ldexpf(p[u], -e);
            pv[u] = ldexpf(pv[u], -e);
          }
        }
        // rescale by each row's factor (1 where the reference stays); the accumulator
        // rows 4q + e of a lane belong to other rows than its own, so every lane takes
        // part (a uniform step: the factors come from the lanes n == row)
        const float f = (m_ref != -INFINITY && m_new != m_ref) ? exp2f(m_ref - m_new) : 1.f;
        l_run *= f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fe = __shfl(f, 4 * q + e);
#pragma unroll
          for (int t = 0; t < 8; ++t) oacc[t][e] *= fe;
        }
        m_ref = m_new;
        thr = (m_ref == -INFINITY) ? -INFINITY : (m_ref + kLazyT) / xs;
      }
    }
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // ---- p * nu_V split into binary16 high and low parts; A-row n < 8: high parts of
    //      row n, A-row n >= 8: low parts of row 15 - n
    H8 hv, lv;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto hh = __builtin_amdgcn_cvt_pkrtz(pv[2 * k], pv[2 * k + 1]);
      const auto ll = __builtin_amdgcn_cvt_pkrtz(pv[2 * k] - (float)hh[0], pv[2 * k + 1] - (float)hh[1]);
      hv.u[k] = __builtin_bit_cast(uint32_t, hh);
      lv.u[k] = __builtin_bit_cast(uint32_t, ll);
    }
    H8 pa;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t keep = lo ? lv.u[k] : hv.u[k];
      const uint32_t recv = dpp_row_mirror_u(lo ? hv.u[k] : lv.u[k]);
      pa.u[k] = lo ? recv : keep;
      pa.u[2 + k] = lo ? keep : recv;
    }
    // ---- PV over the 8 value tiles (coordinate 8n + t of the rotated basis), at raised
    //      wave priority so that a wave holding its operands issues its products first
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa.h, dec_dequant8<VB>(sb, DL, vfield<VB>(blk.vw, t)), oacc[t], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    if (more) {
      if constexpr (PAGED) {
        dec_load_v<VB, KWL>(blk, page_views(__builtin_amdgcn_readfirstlane(pg_next)), t_next, voff_v);
        pg_next = page_of(t0 + 2 * kStep);
      } else {
        dec_load_v<VB, KWL>(blk, R, t_next, voff_v);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- epilogue: rows 0..7 = high row + mirrored low row, merged over the waves into
  //      eight pre-weighted slots in the wave areas, then one partial for the segment
  l_run += dpp_row_mirror(l_run);  // the two lanes of a row summed different tokens
  l_run = sum_over_q(l_run);
  // (lane indices again opaque: the merge's addresses stay in the epilogue)
  int tid_x = tid;
  asm volatile("" : "+v"(tid_x));
  const int q_x = (tid_x >> 4) & 3, n_x = tid_x & 15;
  float vrow[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vrow[t][e] = oacc[t][e] + lane_xor48(oacc[t][3 - e], tid_x & 63);
  }
  __syncthreads();  // every wave is done with its key tile
  if (q_x == 0 && n_x < 8) {
    S.om[wave][n_x] = m_ref;
    S.ol[wave][n_x] = l_run;
  }
  __syncthreads();
  float wt[4];  // 2^(m_wave - M) of rows 4 (q_x & 1) + e (the four rows read as one float4)
  {
    const int r4 = 4 * (q_x & 1);
    float4 M = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float4 o = *reinterpret_cast<const float4*>(&S.om[w][r4]);
      M = make_float4(fmaxf(M.x, o.x), fmaxf(M.y, o.y), fmaxf(M.z, o.z), fmaxf(M.w, o.w));
    }
    const float4 mw = *reinterpret_cast<const float4*>(&S.om[wave][r4]);
    // (<= 1; tiny weights may flush)
    wt[0] = (mw.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw.x - M.x);
    wt[1] = (mw.y == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw.y - M.y);
    wt[2] = (mw.z == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw.z - M.z);
    wt[3] = (mw.w == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw.w - M.w);
  }
  if (wave >= 8 && q_x < 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float* dst = slots + ((wave - 8) * 8 + 4 * q_x + e) * kD + 8 * n_x;
      *reinterpret_cast<float4*>(dst) =
          make_float4(wt[e] * vrow[0][e], wt[e] * vrow[1][e], wt[e] * vrow[2][e], wt[e] * vrow[3][e]);
      *reinterpret_cast<float4*>(dst + 4) =
          make_float4(wt[e] * vrow[4][e], wt[e] * vrow[5][e], wt[e] * vrow[6][e], wt[e] * vrow[7][e]);
    }
  }
  __syncthreads();
  if (wave < 8 && q_x < 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float* dst = slots + (wave * 8 + 4 * q_x + e) * kD + 8 * n_x;
      const float4 x0 = *reinterpret_cast<const float4*>(dst), x1 = *reinterpret_cast<const float4*>(dst + 4);
      *reinterpret_cast<float4*>(dst) = make_float4(fmaf(wt[e], vrow[0][e], x0.x), fmaf(wt[e], vrow[1][e], x0.y),
                                                    fmaf(wt[e], vrow[2][e], x0.z), fmaf(wt[e], vrow[3][e], x0.w));
      *reinterpret_cast<float4*>(dst + 4) = make_float4(fmaf(wt[e], vrow[4][e], x1.x), fmaf(wt[e], vrow[5][e], x1.y),
                                                        fmaf(wt[e], vrow[6][e], x1.z), fmaf(wt[e], vrow[7][e], x1.w));
    }
  }
  __syncthreads();
  if (tid_x < 8 * (kD / 4)) {
    const int r = tid_x >> 5, c4 = tid_x & 31;
    const int id = S.row_id[r];
    if (id >= 0) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, S.om[w][r]);
      float l = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
          const float mw = S.om[w][r];
          l = fmaf((mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M), S.ol[w][r], l);
        }
      }
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(slots + (i * 8 + r) * kD + 4 * c4);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
      float* dst = a.partials + ((size_t)(wg + S.sk_tile) * 8 + r) * kPS;
      *reinterpret_cast<float4*>(dst + 4 + 4 * c4) = acc;
      if (c4 == 0) *reinterpret_cast<float4*>(dst) = make_float4(M, l, 0.f, 0.f);
    }
  }
  __syncthreads();  // the next segment rewrites the wave areas, rows and query operands
  }
}



// ============================================================================
// Phase 2: per row, log-sum-exp merge of its chunk partials, then
// o = Pi_V^T o_rot / sqrt(128) (value reconstruction nu * Pi_V^T C[code] / sqrt(128)).
// ============================================================================

struct MergeArgs {
  const DevHead* heads;    // this layer's heads (Hadamard value rotations)
  const float* vrot_t;     // Pi_V^T of the layer's KV heads, 128 x 128 each, consecutive
  const float* partials;
  const int32_t* seq_len;
  float* out;
  int64_t pos0;
  int32_t n_q, g, n_chunks, chunk, prefill, max_len;
  int32_t win, n_sink, n_recent;  // fp16 window: its split is the last slot
  int32_t batch, n_kv, tiles_per_kv, n_tiles, sk_G;  // decode: the partials' segments (AttnArgs)
  const int4* tile_info;                             // decode: (w0, segments, units) per tile
};

// Four workgroups (256 threads each) per row, one per quarter of the output coordinates:
// thread (float4 column c4, chunk slice ks) loads the accumulators of chunks ks, ks + 8,
// ... together with their (m, l), and thread (output i of the quarter, eighth e) its
// 16 entries of row i of Pi_V^T, in one round; then M = max m, weights 2^(m - M), the
// weighted sums over the slices, normalisation by L sqrt(128) and the quarter's outputs
// of the inverse rotation (eighths added by lane shuffles). Each quarter repeats the
// merge of all 128 accumulator columns and reads only its 16 KB of Pi_V^T.
constexpr int kMergeRegs = 16;  // chunks per thread kept in registers (128 splits in one round)
__global__ void __launch_bounds__(256) attn_merge_kernel(MergeArgs a) {
  __shared__ float4 red[8][32];
  __shared__ float sm[8], sl[8];
  __shared__ float orot[kD];
  __shared__ float opart[2][kD];
  const int row = blockIdx.x, oq = blockIdx.y;
  const int tid = threadIdx.x;
  const int c4 = tid & 31, ks = tid >> 5;
  const int hq = row % a.n_q;
  int len;
  if (a.prefill) len = (int)(a.pos0 + row / a.n_q + 1);
  else len = min(max(a.seq_len[row / a.n_q], 0), a.max_len);
  const int len_p = a.win ? packed_end(len, a.n_sink, a.n_recent) : len;
  // the row's partials: prefill, one per split of its row; decode, one per segment of the
  // partials' workgroups on its row tile, then the window's
  int nv, first = 0, tile = 0, r8 = 0, w0 = 0;
  long long U = 0;
  if (a.prefill) {
    nv = (len_p + a.chunk - 1) / a.chunk;
  } else {
    const int seq = row / a.n_q, f = hq % a.g;
    tile = (seq * a.n_kv + hq / a.g) * a.tiles_per_kv + f / 8;
    r8 = f & 7;
    const int4 inf = a.tile_info[tile];  // (written only for tiles with blocks)
    const int nb = (len_p + 31) >> 5;
    int nseg = 0;
    if (nb > 0) {
      w0 = inf.x;
      first = w0 + tile;
      nseg = inf.y;
      U = (long long)(((unsigned long long)(unsigned)inf.w << 32) | (unsigned)inf.z);
    }
    nv = nseg + a.win;
  }
  auto part = [&](int k) -> const float* {
    if (a.prefill) return a.partials + ((size_t)row * a.n_chunks + k) * kPS;
    const int sg = (a.win && k == nv - 1) ? a.sk_G + a.n_tiles + tile : first + k;
    return a.partials + ((size_t)sg * 8 + r8) * kPS;
  };
  // (with at least as many units as workgroups every workgroup has some: no division)
  const bool all_live = a.prefill || (long long)a.sk_G <= U;
  auto live = [&](int k) { return all_live || (a.win && k == nv - 1) || sk_live(w0 + k, a.sk_G, U); };
  // inverse rotation operand: thread (output oi of this quarter, eighth e) holds
  // Pi_V^T[oi][16 e .. + 15] (none for a Hadamard Pi_V, applied as a transform by the
  // first quarter alone)
  const DevHead* __restrict__ hp = a.heads + hq / a.g;
  const bool had = hp->v_hadamard != 0;
  if (had && oq != 0) return;
  const int nqw = gridDim.y;  // workgroups per row: 4 (one quarter each) or 1 (all four)
  const int oe = tid & 7;
  float4 pvt[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qo = oq + j * nqw, oi = 32 * qo + (tid >> 3);
    const float4* pt = reinterpret_cast<const float4*>(a.vrot_t + (size_t)(hq / a.g) * kD * kD + (size_t)oi * kD + 16 * oe);
#pragma unroll
    for (int u = 0; u < 4; ++u) pvt[j][u] = (had || qo >= 4) ? make_float4(0.f, 0.f, 0.f, 0.f) : pt[u];
  }
  float mk[kMergeRegs], lk[kMergeRegs];
  float4 xk[kMergeRegs];
#pragma unroll
  for (int u = 0; u < kMergeRegs; ++u) {
    const int k = ks + 8 * u;
    mk[u] = -INFINITY;
    lk[u] = 0.f;
    xk[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < nv && live(k)) {
      const float2 ml = *reinterpret_cast<const float2*>(part(k));
      mk[u] = ml.x;
      lk[u] = ml.y;
      xk[u] = *reinterpret_cast<const float4*>(part(k) + 4 + 4 * c4);
    }
  }
  float ms = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMergeRegs; ++u) ms = fmaxf(ms, mk[u]);
  for (int k = ks + 8 * kMergeRegs; k < nv; k += 8)
    if (live(k)) ms = fmaxf(ms, part(k)[0]);
  if (c4 == 0) sm[ks] = ms;
  __syncthreads();
  float M = sm[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) M = fmaxf(M, sm[w]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u) {
      const float w = (mk[u] == -INFINITY) ? 0.f : exp2f(mk[u] - M);
      acc.x = fmaf(w, xk[u].x, acc.x);
      acc.y = fmaf(w, xk[u].y, acc.y);
      acc.z = fmaf(w, xk[u].z, acc.z);
      acc.w = fmaf(w, xk[u].w, acc.w);
      l = fmaf(w, lk[u], l);
    }
    for (int k = ks + 8 * kMergeRegs; k < nv; k += 8) {  // more than 128 partials
      if (!live(k)) continue;
      const float2 ml = *reinterpret_cast<const float2*>(part(k));
      const float4 x = *reinterpret_cast<const float4*>(part(k) + 4 + 4 * c4);
      const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
      l = fmaf(w, ml.y, l);
    }
  }
  red[ks][c4] = acc;
  if (c4 == 0) sl[ks] = l;
  __syncthreads();
  if (tid < 32) {
    float4 s = red[0][tid];
    float L = sl[0];
#pragma unroll
    for (int k2 = 1; k2 < 8; ++k2) {
      const float4 y = red[k2][tid];
      s.x += y.x;
      s.y += y.y;
      s.z += y.z;
      s.w += y.w;
      L += sl[k2];
    }
    const float f = L > 0.f ? 0.08838834764831845f / L : 0.f;  // 1 / (L sqrt(128))
    orot[4 * tid] = s.x * f;
    orot[4 * tid + 1] = s.y * f;
    orot[4 * tid + 2] = s.z * f;
    orot[4 * tid + 3] = s.w * f;
  }
  __syncthreads();
  if (had) {  // o = s * (c H o_rot)
    const float y = wht128(tid < kD ? orot[tid] : 0.f, tid & (kD - 1), tid < kD, opart[0]);
    if (tid < kD) a.out[(size_t)row * kD + tid] = hp->vsign[tid] * kInvSqrt128 * y;
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qo = oq + j * nqw, oi = 32 * qo + (tid >> 3);
    if (qo >= 4) break;
    float o = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 x = *reinterpret_cast<const float4*>(&orot[16 * oe + 4 * u]);
      o = fmaf(pvt[j][u].x, x.x, o);
      o = fmaf(pvt[j][u].y, x.y, o);
      o = fmaf(pvt[j][u].z, x.z, o);
      o = fmaf(pvt[j][u].w, x.w, o);
    }
    o += __shfl_xor(o, 1);
    o += __shfl_xor(o, 2);
    o += __shfl_xor(o, 4);
    if (oe == 0) a.out[(size_t)row * kD + oi] = o;
  }
}

// Merge for up to 8 splits per row: four workgroups (256 threads) per row tile (the rows
// of one sequence and KV head, as in the partials grid), one per quarter of the output
// coordinates, so that each quarter of Pi_V^T is read once per tile. Thread (row r,
// float4 column c4) merges its row's splits in one round of loads; then thread (output
// i of the quarter, eighth e) forms its eighth of the inverse rotation for all 8 rows,
// and lane shuffles add the eighths.
constexpr int kMergeTileChunks = 8;
struct MergeTileArgs {
  const DevHead* heads;    // this layer's heads (Hadamard value rotations)
  const float* vrot_t;     // Pi_V^T of the layer's KV heads, 128 x 128 each, consecutive
  const float* partials;
  const int32_t* seq_len;
  float* out;
  int64_t pos0;
  int32_t n_q, g, n_kv, tiles_per_kv, n_tok, n_chunks, chunk, prefill, max_len, seq;
  int32_t win, n_sink, n_recent;  // fp16 window: its split is the last slot
  int32_t batch, n_tiles, sk_G;   // decode: the partials' segments (AttnArgs)
  const int4* tile_info;          // decode: (w0, segments, units) per tile
};

__global__ void __launch_bounds__(256) attn_merge_tile_kernel(MergeTileArgs a) {
  __shared__ float4 accs[8][kD / 4];
  __shared__ int32_t rid[8];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x, oq = blockIdx.y;
  int seq, h, tr;
  if (a.prefill) {
    h = tile / a.tiles_per_kv;
    tr = tile - h * a.tiles_per_kv;
    seq = a.seq;
  } else {
    seq = tile / (a.n_kv * a.tiles_per_kv);
    const int rem = tile - seq * a.n_kv * a.tiles_per_kv;
    h = rem / a.tiles_per_kv;
    tr = rem - h * a.tiles_per_kv;
  }
  // the inverse rotation operand first: thread (output oi of this quarter, eighth e)
  // holds Pi_V^T[oi][16 e .. + 15] (none for a Hadamard Pi_V, applied as a transform by
  // the first quarter alone)
  const DevHead* __restrict__ hp = a.heads + h;
  const bool had = hp->v_hadamard != 0;
  if (had && oq != 0) return;
  const int nqw = gridDim.y;  // workgroups per tile: 4 (one quarter each) or 1 (all four)
  const int oe = tid & 7;
  float4 pvt[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qo = oq + j * nqw, oi = 32 * qo + (tid >> 3);
    const float4* pt = reinterpret_cast<const float4*>(a.vrot_t + (size_t)h * kD * kD + (size_t)oi * kD + 16 * oe);
#pragma unroll
    for (int u = 0; u < 4; ++u) pvt[j][u] = (had || qo >= 4) ? make_float4(0.f, 0.f, 0.f, 0.f) : pt[u];
  }
  // decode: the partials of this row tile, one per segment of the partials' workgroups on
  // it, then the window's
  int first = 0, nseg = 0, w0 = 0;
  long long U = 0;
  if (!a.prefill) {
    const int4 inf = a.tile_info[tile];  // (written only for tiles with blocks)
    const int nb = seq_blocks(a.seq_len, seq, a.max_len, a.win, a.n_sink, a.n_recent);
    if (nb > 0) {
      w0 = inf.x;
      first = w0 + tile;
      nseg = inf.y;
      U = (long long)(((unsigned long long)(unsigned)inf.w << 32) | (unsigned)inf.z);
    }
  }
  // row r of the tile: global row id (-1 if absent) and visible length
  const int r = tid >> 5, c4 = tid & 31;
  const int f = tr * 8 + r;
  int id = -1, len = 0;
  if (a.prefill) {
    if (f < a.n_tok * a.g) {
      const int t = f / a.g;
      id = t * a.n_q + h * a.g + (f - t * a.g);
      len = (int)(a.pos0 + t + 1);
    }
  } else if (f < a.g) {
    id = seq * a.n_q + h * a.g + f;
    len = min(max(a.seq_len[seq], 0), a.max_len);
  }
  if (c4 == 0) rid[r] = id;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  if (id >= 0) {
    const int nv = a.prefill ? min(a.n_chunks, (len + a.chunk - 1) / a.chunk) : nseg + a.win;
    auto part = [&](int k) -> const float* {
      if (a.prefill) return a.partials + ((size_t)id * a.n_chunks + k) * kPS;
      const int sg = (a.win && k == nv - 1) ? a.sk_G + a.n_tiles + tile : first + k;
      return a.partials + ((size_t)sg * 8 + r) * kPS;
    };
    // (with at least as many units as workgroups every workgroup has some: no division)
    const bool all_live = a.prefill || (long long)a.sk_G <= U;
    auto live = [&](int k) { return all_live || (a.win && k == nv - 1) || sk_live(w0 + k, a.sk_G, U); };
    float mk[kMergeTileChunks], lk[kMergeTileChunks];
    float4 xk[kMergeTileChunks];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeTileChunks; ++k) {
      mk[k] = -INFINITY;
      lk[k] = 0.f;
      xk[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < nv && live(k)) {
        const float2 ml = *reinterpret_cast<const float2*>(part(k));
        mk[k] = ml.x;
        lk[k] = ml.y;
        xk[k] = *reinterpret_cast<const float4*>(part(k) + 4 + 4 * c4);
      }
      M = fmaxf(M, mk[k]);
    }
    for (int k = kMergeTileChunks; k < nv; ++k)
      if (live(k)) M = fmaxf(M, part(k)[0]);
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kMergeTileChunks; ++k) {
        const float w = (mk[k] == -INFINITY) ? 0.f : exp2f(mk[k] - M);
        acc.x = fmaf(w, xk[k].x, acc.x);
        acc.y = fmaf(w, xk[k].y, acc.y);
        acc.z = fmaf(w, xk[k].z, acc.z);
        acc.w = fmaf(w, xk[k].w, acc.w);
        L = fmaf(w, lk[k], L);
      }
      for (int k = kMergeTileChunks; k < nv; ++k) {  // more partials than registers
        if (!live(k)) continue;
        const float2 ml = *reinterpret_cast<const float2*>(part(k));
        const float4 x = *reinterpret_cast<const float4*>(part(k) + 4 + 4 * c4);
        const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
        acc.x = fmaf(w, x.x, acc.x);
        acc.y = fmaf(w, x.y, acc.y);
        acc.z = fmaf(w, x.z, acc.z);
        acc.w = fmaf(w, x.w, acc.w);
        L = fmaf(w, ml.y, L);
      }
    }
  }
  const float sc = L > 0.f ? 0.08838834764831845f / L : 0.f;  // 1 / (L sqrt(128))
  if (had) {
    // o = s * (c H o_rot): the thread holds elements 4 c4 .. + 3 of its row; strides 1, 2
    // in registers, 4 .. 64 across the row's 32 lanes
    float v[4] = {acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc};
    const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    v[0] = a0 + a2;
    v[1] = a1 + a3;
    v[2] = a0 - a2;
    v[3] = a1 - a3;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = __shfl_xor(v[j], m);
        v[j] = (c4 & m) ? y - v[j] : v[j] + y;
      }
    }
    if (id >= 0) {
      const float* sg = hp->vsign + 4 * c4;
      *reinterpret_cast<float4*>(a.out + (size_t)id * kD + 4 * c4) =
          make_float4(sg[0] * kInvSqrt128 * v[0], sg[1] * kInvSqrt128 * v[1], sg[2] * kInvSqrt128 * v[2],
                      sg[3] * kInvSqrt128 * v[3]);
    }
    return;
  }
  accs[r][c4] = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qo = oq + j * nqw, oi = 32 * qo + (tid >> 3);
    if (qo >= 4) break;
    float o[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) o[rr] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float4 x = accs[rr][4 * oe + u];
        o[rr] = fmaf(pvt[j][u].x, x.x, o[rr]);
        o[rr] = fmaf(pvt[j][u].y, x.y, o[rr]);
        o[rr] = fmaf(pvt[j][u].z, x.z, o[rr]);
        o[rr] = fmaf(pvt[j][u].w, x.w, o[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      o[rr] += __shfl_xor(o[rr], 1);
      o[rr] += __shfl_xor(o[rr], 2);
      o[rr] += __shfl_xor(o[rr], 4);
      const int orow = rid[rr];
      if (oe == 0 && orow >= 0) a.out[(size_t)orow * kD + oi] = o[rr];
    }
  }
}

// ============================================================================
// host helpers
// ============================================================================

bool check_device_plan(const gtq_plan* p, const char* fn, gtq_status* st) {
  if (!p) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": plan is NULL");
    return false;
  }
  if (!p->d_heads) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": plan was created host-only");
    return false;
  }
  return true;
}

bool check_cache(const gtq_plan* p, const gtq_cache_view* c, const char* fn, gtq_status* st) {
  if (!c || !c->k_codes || !c->k_norms || !c->v_codes || !c->v_norms) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": cache view or one of its buffers is NULL");
    return false;
  }
  if (c->batch < 1 || c->capacity < 1 || c->capacity % GTQ_SEQ_ALIGN) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": cache batch >= 1 and capacity a positive multiple of 32");
    return false;
  }
  if (c->block_table) {
    const int P = c->page_tokens;
    if (P < 32 || (P & (P - 1)) || P > kMaxCapacity || c->n_pages < 1 || c->table_stride < 1 ||
        c->capacity > (int64_t)c->table_stride * P) {
      *st = fail(GTQ_EINVAL, std::string(fn) + ": paged cache needs page_tokens a power of two in [32, 2^25], "
                                             "n_pages >= 1, table_stride >= 1, capacity <= table_stride * page_tokens");
      return false;
    }
  } else if (c->capacity > kMaxCapacity) {  // one (sequence, KV head) slice stays under 2 GiB
    *st = fail(GTQ_EUNSUPPORTED, std::string(fn) + ": capacity above 2^25 tokens");
    return false;
  }
  (void)p;
  return true;
}

PageMap page_map(const gtq_cache_view* c) {
  PageMap m{};
  if (c->block_table) {
    m.table = c->block_table;
    m.P = c->page_tokens;
    m.log2P = __builtin_ctz((unsigned)c->page_tokens);
    m.n_pages = c->n_pages;
    m.tstride = c->table_stride;
  }
  return m;
}

void fill_append_args(const gtq_plan* p, int layer, const gtq_cache_view* c, const float* k, const float* v,
                      AppendArgs& a) {
  a.heads = p->d_heads + (size_t)layer * p->n_kv;
  a.rot = p->d_rot;
  a.rsplit = p->d_rsplit;
  a.cb = p->d_cb;
  a.k_codes = c->k_codes;
  a.k_norms = c->k_norms;
  a.v_codes = c->v_codes;
  a.v_norms = c->v_norms;
  a.k = k;
  a.v = v;
  a.overflow = p->d_overflow;
  a.capacity = c->capacity;
  a.batch = c->batch;
  a.n_kv = p->n_kv;
  a.k_words = p->k_words;
  a.v_bits = p->v_bits;
  a.nc = (p->flags & GTQ_PLAN_NORM_CORRECT) ? 1 : 0;
  a.pm = page_map(c);
}

gtq_status launch_append(const gtq_plan* p, int layer, const gtq_cache_view* c, const float* k,
                         const float* v, const int32_t* seq_idx, const int64_t* slot, int32_t seq,
                         int64_t pos0, int64_t n_tok, bool chunk, hipStream_t stream) {
  AppendArgs a{};
  a.heads = p->d_heads + (size_t)layer * p->n_kv;
  a.rot = p->d_rot;
  a.rsplit = p->d_rsplit;
  a.cb = p->d_cb;
  a.k_codes = c->k_codes;
  a.k_norms = c->k_norms;
  a.v_codes = c->v_codes;
  a.v_norms = c->v_norms;
  a.k = k;
  a.v = v;
  a.seq_idx = seq_idx;
  a.slot = slot;
  a.overflow = p->d_overflow;
  a.capacity = c->capacity;
  a.n_tok = n_tok;
  a.pos0 = pos0;
  a.seq = seq;
  a.batch = c->batch;
  a.n_kv = p->n_kv;
  a.k_words = p->k_words;
  a.v_bits = p->v_bits;
  a.nc = (p->flags & GTQ_PLAN_NORM_CORRECT) ? 1 : 0;
  a.pm = page_map(c);
  // QJL plans append through the per-token kernel (chunks included: no index arrays)
  if (!chunk || (p->flags & GTQ_PLAN_QJL)) {
    if (n_tok > 0x7FFFFFFF) return fail(GTQ_EUNSUPPORTED, "gtq_quantize_append: too many tokens");
    if (n_tok == 0) return ok();
    hipLaunchKernelGGL(append_token_kernel, dim3((unsigned)n_tok, p->n_kv, append_roles(n_tok * p->n_kv)), dim3(1024),
                       0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "gtq append: launch");
    return ok();
  }
  a.n_tok = n_tok;
  a.pos0 = pos0;
  a.seq = seq;
  const int64_t s_begin = pos0 & ~(int64_t)(GTQ_VBLOCK - 1);
  const int64_t n_tiles = (pos0 + n_tok - s_begin + kAppTile - 1) / kAppTile;
  // one round of workgroups, two per compute unit (512), each over several tiles with the
  // next tile's inputs in flight
  const int64_t per_head = std::max<int64_t>(1, 512 / (2 * (int64_t)p->n_kv));
  const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(n_tiles, per_head));
  hipLaunchKernelGGL(append_gemm_kernel, dim3((unsigned)(gx * p->n_kv * 2)), dim3(kAppThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq append: launch");
  return ok();
}

int auto_chunk(int64_t max_len, int64_t tiles, int64_t kRound) {
  // one round of workgroups (one per compute unit), at least 4 splits per row tile so
  // that ragged batches balance; splits of whole rounds of the main loop (waves x 32
  // tokens: 16 waves for the decode tiles, 8 for the prefill tiles)
  int64_t target = std::max<int64_t>(4, kTargetWG / std::max<int64_t>(1, tiles));
  target = std::min<int64_t>(kMaxChunks, target);
  int64_t ch = (max_len + target - 1) / target;
  ch = ((ch + kRound - 1) / kRound) * kRound;
  return (int)std::max<int64_t>(kRound, ch);
}

// workspace: the tiles' QK B operands, then the partials
// rotated-query operands of n_tiles row tiles of rt rows (8 KB per 8 rows)
// (followed by one float per tile: the factor 2^sq that undoes the operands' range scaling)
// (QJL plans: then the residual sketch's operands, 4 KB per tile)
size_t attn_qb_bytes(int64_t n_tiles, int rt, bool qjl = false) {
  return (size_t)n_tiles * (rt / 8) * kQB * sizeof(uint4) + ((size_t)n_tiles * 4 + 15) / 16 * 16 +
         (qjl ? (size_t)n_tiles * 256 * sizeof(uint4) : 0);
}
size_t attn_ws_bytes(int64_t rows, int64_t n_chunks, size_t qb_bytes) {
  return qb_bytes + (size_t)rows * n_chunks * kPS * 4;
}
// decode: one 8-row partial per (workgroup, tile) segment, w + t < sk_G + n_tiles, then
// one per tile for the window's split; then the tiles' merge pointers (16 bytes each)
size_t decode_part_bytes(int64_t n_tiles, int sk_G) { return (size_t)(sk_G + 2 * n_tiles) * 8 * kPS * 4; }
size_t decode_ws_bytes(int64_t n_tiles, int sk_G, size_t qb_bytes) {
  return qb_bytes + decode_part_bytes(n_tiles, sk_G) + (size_t)n_tiles * 16;
}

struct AttnLaunch {
  int64_t rows;
  int sk_G;                // decode: partials workgroups (each an equal share of the batch's units)
  int rt;                  // rows per partials tile: 8 (decode) or 16 (prefill)
  int tiles_per_kv;        // partials / query-rotation tiles
  int n_tiles;
  int merge_tiles_per_kv;  // 8-row tiles of the merge
  int merge_n_tiles;
  size_t qb_bytes;         // rotated-query operands at the start of the workspace
  int chunk;
  int n_chunks;
};

void fill_attn_args(const gtq_plan* p, int layer, const gtq_cache_view* c, AttnArgs& aa, const AttnLaunch& L,
                    void* ws) {
  aa.heads = p->d_heads + (size_t)layer * p->n_kv;
  aa.rot = p->d_rot;
  aa.cb = p->d_cb;
  aa.k_codes = c->k_codes;
  aa.k_norms = c->k_norms;
  aa.v_codes = c->v_codes;
  aa.v_norms = c->v_norms;
  aa.qb = reinterpret_cast<uint4*>(ws);
  aa.tile_xs = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (size_t)L.n_tiles * (L.rt / 8) * kQB * sizeof(uint4));
  aa.qjl = (p->flags & GTQ_PLAN_QJL) ? 1 : 0;
  aa.mse_words = 2 * p->k_budget / 32;
  aa.qjl_qb = aa.qjl ? reinterpret_cast<uint4*>(reinterpret_cast<char*>(aa.tile_xs) + ((size_t)L.n_tiles * 4 + 15) / 16 * 16)
                     : nullptr;
  aa.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + L.qb_bytes);
  aa.tile_info = L.rt == 8 ? reinterpret_cast<int4*>(reinterpret_cast<char*>(ws) + L.qb_bytes +
                                                     decode_part_bytes(L.n_tiles, L.sk_G))
                           : nullptr;
  aa.capacity = c->capacity;
  aa.n_kv = p->n_kv;
  aa.n_q = p->n_q;
  aa.g = p->n_q / p->n_kv;
  aa.k_words = p->k_words;
  aa.tiles_per_kv = L.tiles_per_kv;
  aa.chunk = L.chunk;
  aa.n_chunks = L.n_chunks;
  aa.batch = (int32_t)(L.rows / p->n_q);
  aa.n_tiles = L.n_tiles;
  aa.sk_G = L.sk_G;
  aa.pm = page_map(c);
  aa.nkb_max = 0;
  for (int h = 0; h < p->n_kv; ++h) aa.nkb_max = std::max(aa.nkb_max, (int32_t)p->heads[(size_t)layer * p->n_kv + h].nkb);
}

gtq_status launch_qrot(AttnArgs& aa, const AttnLaunch& L, const float* q, float scale, hipStream_t stream) {
  aa.q = q;
  aa.qscale = scale * LOG2E_F;
  if (L.rt == 16)
    hipLaunchKernelGGL(attn_qrot_kernel<16>, dim3(L.n_tiles), dim3(64 * kQrotWaves), 0, stream, aa);
  else
    hipLaunchKernelGGL(attn_qrot_kernel<8>, dim3(L.n_tiles), dim3(64 * kQrotWaves), 0, stream, aa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq attention query rotation: launch");
  return ok();
}

// decode tiles: attn_decode_kernel<VB, KWL, N1, N4> with the layer's specialized slot
// counts (N1 <= 3, N4 <= min(3, 4 - N1))
template <int VB, int KWL>
void launch_decode(dim3 grid, int n1, int n4, const AttnArgs& aa, hipStream_t stream) {
  if (aa.qjl) {  // QJL plans: every slot through the generic path, and the sketch
    if (aa.pm.table) hipLaunchKernelGGL((attn_decode_kernel<VB, KWL, 0, 0, true, true>), grid, dim3(kDecThreads), 0, stream, aa);
    else hipLaunchKernelGGL((attn_decode_kernel<VB, KWL, 0, 0, false, true>), grid, dim3(kDecThreads), 0, stream, aa);
    return;
  }
  if (aa.pm.table) {  // paged caches: every slot through the generic path
    hipLaunchKernelGGL((attn_decode_kernel<VB, KWL, 0, 0, true, false>), grid, dim3(kDecThreads), 0, stream, aa);
    return;
  }
#define GTQ_DEC(A, B) hipLaunchKernelGGL((attn_decode_kernel<VB, KWL, A, B, false, false>), grid, dim3(kDecThreads), 0, stream, aa)
  switch (n1 * 4 + n4) {
    case 0: GTQ_DEC(0, 0); break;
    case 1: GTQ_DEC(0, 1); break;
    case 2: GTQ_DEC(0, 2); break;
    case 3: GTQ_DEC(0, 3); break;
    case 4: GTQ_DEC(1, 0); break;
    case 5: GTQ_DEC(1, 1); break;
    case 6: GTQ_DEC(1, 2); break;
    case 7: GTQ_DEC(1, 3); break;
    case 8: GTQ_DEC(2, 0); break;
    case 9: GTQ_DEC(2, 1); break;
    case 10: GTQ_DEC(2, 2); break;
    case 12: GTQ_DEC(3, 0); break;
    default: GTQ_DEC(3, 1); break;
  }
#undef GTQ_DEC
}

gtq_status launch_partials(const gtq_plan* p, int layer, AttnArgs& aa, const AttnLaunch& L, hipStream_t stream) {
  if (p->k_words > 16) return fail(GTQ_EUNSUPPORTED, "gtq attention: more than 16 key code words per token");
  dim3 grid(L.n_chunks - aa.win, L.n_tiles);  // (the window's split comes from its own launch)
  const bool wide = p->k_words > 8;  // key words per lane: 4 (k_words <= 8) or 8
  if (L.rt == 8) {
    grid = dim3((unsigned)L.sk_G);
    const int n1 = p->layer_n1[layer], n4 = p->layer_n4[layer];
#define GTQ_DECV(VB) \
  if (wide) launch_decode<VB, 8>(grid, n1, n4, aa, stream); else launch_decode<VB, 4>(grid, n1, n4, aa, stream)
    switch (p->v_bits) {
      case 1: GTQ_DECV(1); break;
      case 2: GTQ_DECV(2); break;
      case 3: GTQ_DECV(3); break;
      default: GTQ_DECV(4); break;
    }
#undef GTQ_DECV
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "gtq attention partials: launch");
    return ok();
  }
  // K-blocks per head: sum_g ceil(d_g / 32), 4..7 for four groups; the kernel runs the
  // layer's largest count (extra K-blocks of a head have zero query operands)
  const int nkb = aa.nkb_max;
  if (nkb < 4 || nkb > 7) return fail(GTQ_EUNSUPPORTED, "gtq attention: K-block count outside 4..7");
#define GTQ_LAUNCH4(VB, KWL, NKB, PG) \
  hipLaunchKernelGGL((attn_partials_kernel<VB, KWL, NKB, 16, PG>), grid, dim3(kThreads), 0, stream, aa)
#define GTQ_LAUNCH3(VB, KWL, NKB) \
  if (aa.pm.table) { GTQ_LAUNCH4(VB, KWL, NKB, true); } else { GTQ_LAUNCH4(VB, KWL, NKB, false); }
#define GTQ_LAUNCH2(VB, KWL)                  \
  switch (nkb) {                              \
    case 4: GTQ_LAUNCH3(VB, KWL, 4); break;   \
    case 5: GTQ_LAUNCH3(VB, KWL, 5); break;   \
    case 6: GTQ_LAUNCH3(VB, KWL, 6); break;   \
    default: GTQ_LAUNCH3(VB, KWL, 7); break;  \
  }
#define GTQ_LAUNCH(VB) \
  if (wide) { GTQ_LAUNCH2(VB, 8) } else { GTQ_LAUNCH2(VB, 4) }
  switch (p->v_bits) {
    case 1: GTQ_LAUNCH(1) break;
    case 2: GTQ_LAUNCH(2) break;
    case 3: GTQ_LAUNCH(3) break;
    default: GTQ_LAUNCH(4) break;
  }
#undef GTQ_LAUNCH
#undef GTQ_LAUNCH2
#undef GTQ_LAUNCH3
#undef GTQ_LAUNCH4
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq attention partials: launch");
  return ok();
}

// merge workgroups per row (tile): one per quarter of the inverse rotation while few rows
// (tiles) leave most compute units idle, else one
inline unsigned merge_quarters(int64_t n) { return n <= 256 ? 4u : 1u; }

gtq_status launch_merge(const gtq_plan* p, int layer, const AttnLaunch& L, const int32_t* seq_len,
                        int64_t pos0, int prefill, int max_len, float* out, const void* ws,
                        hipStream_t stream, const gtq_window_view* w = nullptr) {
  const float* vrot_t = p->d_rot + p->heads[(size_t)layer * p->n_kv].vrot_t_off;
  const float* partials = reinterpret_cast<const float*>(reinterpret_cast<const char*>(ws) + L.qb_bytes);
  const int4* tile_info = prefill ? nullptr
                                  : reinterpret_cast<const int4*>(reinterpret_cast<const char*>(ws) + L.qb_bytes +
                                                                  decode_part_bytes(L.n_tiles, L.sk_G));
  // one workgroup per row tile when few partials per row are expected (prefill: at most
  // kMergeTileChunks splits; decode: about sk_G / n_tiles + 2 segments per tile)
  const bool tile_merge = prefill ? L.n_chunks <= kMergeTileChunks : L.sk_G <= 4 * L.n_tiles;
  if (tile_merge) {
    MergeTileArgs mt{p->d_heads + (size_t)layer * p->n_kv, vrot_t, partials, seq_len, out, pos0, p->n_q, p->n_q / p->n_kv, p->n_kv, L.merge_tiles_per_kv,
                     (int32_t)(L.rows / p->n_q), L.n_chunks, L.chunk, prefill, max_len, 0};
    if (w) {
      mt.win = 1;
      mt.n_sink = w->n_sink;
      mt.n_recent = w->n_recent;
    }
    mt.batch = (int32_t)(L.rows / p->n_q);
    mt.n_tiles = L.n_tiles;
    mt.sk_G = L.sk_G;
    mt.tile_info = tile_info;
    hipLaunchKernelGGL(attn_merge_tile_kernel, dim3((unsigned)L.merge_n_tiles, merge_quarters(L.merge_n_tiles)),
                       dim3(256), 0, stream, mt);
  } else {  // one workgroup per row
    MergeArgs ma{p->d_heads + (size_t)layer * p->n_kv, vrot_t, partials, seq_len, out, pos0, p->n_q, p->n_q / p->n_kv, L.n_chunks, L.chunk, prefill,
                 max_len};
    if (w) {
      ma.win = 1;
      ma.n_sink = w->n_sink;
      ma.n_recent = w->n_recent;
    }
    ma.batch = (int32_t)(L.rows / p->n_q);
    ma.n_kv = p->n_kv;
    ma.tiles_per_kv = L.merge_tiles_per_kv;
    ma.n_tiles = L.n_tiles;
    ma.sk_G = L.sk_G;
    ma.tile_info = tile_info;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)L.rows, merge_quarters(L.rows)), dim3(256), 0, stream, ma);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq attention merge: launch");
  return ok();
}

// ---------------------------------------------------------------- static scratch
// The workspace of gtq_decode_attn_static: a device array of fixed size in the library
// (each device holds its own copy until the process ends). Host code uses only the
// address that hipGetSymbolAddress returns for it on each device, taken once per device
// at plan creation with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

gtq_status scratch_init(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return fail(GTQ_EUNSUPPORTED, "gtq_plan_create: device index too large");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return ok();
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "gtq_plan_create: scratch address");
  g_scratch_ptr[device] = ptr;
  return ok();
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

gtq_status gtq_plan_create(const gtq_plan_desc* desc, gtq_plan** out) {
  if (!out) return fail(GTQ_EINVAL, "gtq_plan_create: out is NULL");
  *out = nullptr;
  gtq_plan* p = new (std::nothrow) gtq_plan();
  if (!p) return fail(GTQ_ENOMEM, "gtq_plan_create: host allocation failed");
  gtq_status st = plan_build_host(desc, p);
  if (st != GTQ_OK) {
    delete p;
    return st;
  }
  if (!(p->flags & GTQ_PLAN_HOST_ONLY)) {
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "gtq_plan_create: no HIP device");
    }
    int n_cu = 0;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, p->device)) != hipSuccess) {
      delete p;
      return hip_fail(e, "gtq_plan_create: device query");
    }
    p->n_cu = std::max(1, n_cu);
    if ((st = scratch_init(p->device)) != GTQ_OK) {
      delete p;
      return st;
    }
    const size_t hb = p->heads.size() * sizeof(DevHead);
    const size_t rb = p->rot.size() * sizeof(float);
    const size_t sb = p->rsplit.size() * sizeof(uint16_t);
    if ((e = hipMalloc(&p->d_heads, hb)) != hipSuccess || (e = hipMalloc(&p->d_rot, rb)) != hipSuccess ||
        (e = hipMalloc(&p->d_rsplit, sb)) != hipSuccess ||
        (e = hipMalloc(&p->d_cb, sizeof(DevCodebook))) != hipSuccess ||
        (e = hipMalloc(&p->d_overflow, sizeof(unsigned long long))) != hipSuccess) {
      gtq_plan_destroy(p);
      return fail(GTQ_ENOMEM, std::string("gtq_plan_create: device allocation failed: ") + hipGetErrorString(e));
    }
    if ((e = hipMemcpy(p->d_heads, p->heads.data(), hb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(p->d_rot, p->rot.data(), rb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(p->d_rsplit, p->rsplit.data(), sb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(p->d_cb, &p->cb, sizeof(DevCodebook), hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemset(p->d_overflow, 0, sizeof(unsigned long long))) != hipSuccess) {
      gtq_plan_destroy(p);
      return hip_fail(e, "gtq_plan_create: upload");
    }
  }
  *out = p;
  return ok();
}

gtq_status gtq_plan_destroy(gtq_plan* p) {
  if (!p) return ok();
  if (p->d_heads || p->d_rot || p->d_rsplit || p->d_cb || p->d_overflow) {
    (void)hipDeviceSynchronize();
    (void)hipFree(p->d_heads);
    (void)hipFree(p->d_rot);
    (void)hipFree(p->d_rsplit);
    (void)hipFree(p->d_cb);
    (void)hipFree(p->d_overflow);
  }
  delete p;
  return ok();
}

gtq_status gtq_plan_overflow_count(const gtq_plan* p, int64_t* out) {
  gtq_status st;
  if (!out) return fail(GTQ_EINVAL, "gtq_plan_overflow_count: out is NULL");
  if (!check_device_plan(p, "gtq_plan_overflow_count", &st)) return st;
  unsigned long long v = 0;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(&v, p->d_overflow, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "gtq_plan_overflow_count");
  *out = (int64_t)v;
  return ok();
}

gtq_status gtq_quantize_append(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                               const float* k, const float* v, const int32_t* seq_idx,
                               const int64_t* slot, int64_t n_tok, void* hip_stream) {
  gtq_status st;
  if (!check_device_plan(plan, "gtq_quantize_append", &st)) return st;
  if (!check_cache(plan, cache, "gtq_quantize_append", &st)) return st;
  if (layer < 0 || layer >= plan->n_layers) return fail(GTQ_EINVAL, "gtq_quantize_append: layer out of range");
  if (n_tok < 0) return fail(GTQ_EINVAL, "gtq_quantize_append: n_tok < 0");
  if (n_tok == 0) return ok();
  if (!k || !v || !seq_idx || !slot) return fail(GTQ_EINVAL, "gtq_quantize_append: NULL input");
  return launch_append(plan, layer, cache, k, v, seq_idx, slot, 0, 0, n_tok, false,
                       (hipStream_t)hip_stream);
}

gtq_status gtq_quantize_append_chunk(const gtq_plan* plan, int32_t layer,
                                     const gtq_cache_view* cache, const float* k, const float* v,
                                     int32_t seq, int64_t pos0, int64_t n_tok, void* hip_stream) {
  gtq_status st;
  if (!check_device_plan(plan, "gtq_quantize_append_chunk", &st)) return st;
  if (!check_cache(plan, cache, "gtq_quantize_append_chunk", &st)) return st;
  if (layer < 0 || layer >= plan->n_layers) return fail(GTQ_EINVAL, "gtq_quantize_append_chunk: layer out of range");
  if (seq < 0 || seq >= cache->batch) return fail(GTQ_EINVAL, "gtq_quantize_append_chunk: seq out of range");
  if (n_tok < 0 || pos0 < 0) return fail(GTQ_EINVAL, "gtq_quantize_append_chunk: negative pos0 or n_tok");
  if (pos0 + n_tok > cache->capacity) return fail(GTQ_ECAPACITY, "gtq_quantize_append_chunk: pos0 + n_tok > capacity");
  if (n_tok == 0) return ok();
  if (!k || !v) return fail(GTQ_EINVAL, "gtq_quantize_append_chunk: NULL input");
  return launch_append(plan, layer, cache, k, v, nullptr, nullptr, seq, pos0, n_tok, true,
                       (hipStream_t)hip_stream);
}

static bool decode_shape(const gtq_plan* p, int32_t batch, int64_t max_len, int32_t chunk,
                         AttnLaunch* L, gtq_status* st, const char* fn, int win = 0) {
  if (max_len < 0) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": max_len < 0");
    return false;
  }
  if (max_len > INT32_MAX) {
    *st = fail(GTQ_EUNSUPPORTED, std::string(fn) + ": max_len too large");
    return false;
  }
  if (chunk < 0 || chunk % kBlk) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": chunk must be 0 or a positive multiple of 32");
    return false;
  }
  const int g = p->n_q / p->n_kv;
  L->rows = (int64_t)batch * p->n_q;
  L->rt = 8;
  L->tiles_per_kv = (g + 7) / 8;
  L->n_tiles = batch * p->n_kv * L->tiles_per_kv;
  L->merge_tiles_per_kv = L->tiles_per_kv;
  L->merge_n_tiles = L->n_tiles;
  L->qb_bytes = attn_qb_bytes(L->n_tiles, L->rt, (p->flags & GTQ_PLAN_QJL) != 0);
  L->chunk = chunk ? chunk : auto_chunk(max_len, L->n_tiles, kBlk * kDecWaves);
  L->n_chunks = (int)std::max<int64_t>(1, (max_len + L->chunk - 1) / L->chunk);
  if (L->n_chunks > kMaxChunks) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": chunk too small (more than 256 splits per sequence)");
    return false;
  }
  // partials workgroups: one per compute unit, or with an explicit chunk as many as the
  // splits of a batch at max_len (chunk / 32 blocks each when every row has max_len)
  const int64_t g_req = chunk ? (int64_t)L->n_tiles * L->n_chunks : (int64_t)p->n_cu;
  if (g_req > (int64_t)1 << 20) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": chunk too small for this batch");
    return false;
  }
  L->sk_G = (int)std::max<int64_t>(1, g_req);
  L->n_chunks += win;  // the fp16 window's split
  return true;
}

gtq_status gtq_decode_workspace_bytes(const gtq_plan* plan, int32_t batch, int64_t max_len,
                                      int32_t chunk, size_t* out) {
  if (!plan || !out) return fail(GTQ_EINVAL, "gtq_decode_workspace_bytes: NULL pointer");
  if (batch < 1) return fail(GTQ_EINVAL, "gtq_decode_workspace_bytes: batch < 1");
  AttnLaunch L;
  gtq_status st;
  if (!decode_shape(plan, batch, max_len, chunk, &L, &st, "gtq_decode_workspace_bytes")) return st;
  *out = decode_ws_bytes(L.n_tiles, L.sk_G, L.qb_bytes);
  return ok();
}

static gtq_status decode_check(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                               int64_t max_len, int32_t chunk, size_t ws_bytes, const void* ws,
                               AttnLaunch* L, const char* fn, int win = 0) {
  gtq_status st;
  if (!check_device_plan(plan, fn, &st)) return st;
  if (!check_cache(plan, cache, fn, &st)) return st;
  if (layer < 0 || layer >= plan->n_layers) return fail(GTQ_EINVAL, std::string(fn) + ": layer out of range");
  if (!ws) return fail(GTQ_EINVAL, std::string(fn) + ": workspace is NULL");
  if (max_len > cache->capacity) return fail(GTQ_ECAPACITY, std::string(fn) + ": max_len > capacity");
  if (!decode_shape(plan, cache->batch, max_len, chunk, L, &st, fn, win)) return st;
  if (ws_bytes < decode_ws_bytes(L->n_tiles, L->sk_G, L->qb_bytes))
    return fail(GTQ_ECAPACITY, std::string(fn) + ": workspace too small");
  return GTQ_OK;
}

gtq_status gtq_decode_rotate_queries(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                     const float* q, int64_t max_len, float softmax_scale, int32_t chunk,
                                     void* workspace, size_t ws_bytes, void* hip_stream) {
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L,
                               "gtq_decode_rotate_queries");
  if (st != GTQ_OK) return st;
  if (!q) return fail(GTQ_EINVAL, "gtq_decode_rotate_queries: q is NULL");
  if (!isfinite(softmax_scale)) return fail(GTQ_EINVAL, "gtq_decode_rotate_queries: softmax_scale not finite");
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.prefill = 0;
  aa.max_len = (int32_t)max_len;
  return launch_qrot(aa, L, q, softmax_scale, (hipStream_t)hip_stream);
}

gtq_status gtq_decode_attn_partials(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                    const int32_t* seq_len, int64_t max_len, int32_t chunk, float* logits,
                                    void* workspace, size_t ws_bytes, void* hip_stream) {
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L,
                               "gtq_decode_attn_partials");
  if (st != GTQ_OK) return st;
  if (!seq_len) return fail(GTQ_EINVAL, "gtq_decode_attn_partials: seq_len is NULL");
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.logits = logits;
  aa.logits_ld = max_len;
  aa.seq_len = seq_len;
  aa.prefill = 0;
  aa.max_len = (int32_t)max_len;
  return launch_partials(plan, layer, aa, L, (hipStream_t)hip_stream);
}

gtq_status gtq_decode_attn_merge(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                 const int32_t* seq_len, int64_t max_len, int32_t chunk, float* out,
                                 const void* workspace, size_t ws_bytes, void* hip_stream) {
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L,
                               "gtq_decode_attn_merge");
  if (st != GTQ_OK) return st;
  if (!seq_len || !out) return fail(GTQ_EINVAL, "gtq_decode_attn_merge: NULL pointer");
  return launch_merge(plan, layer, L, seq_len, 0, 0, (int)max_len, out, workspace, (hipStream_t)hip_stream);
}

gtq_status gtq_decode_attn(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                           const float* q, const int32_t* seq_len, int64_t max_len,
                           float softmax_scale, int32_t chunk, float* out, float* logits,
                           void* workspace, size_t ws_bytes, void* hip_stream) {
  if (!out) return fail(GTQ_EINVAL, "gtq_decode_attn: out is NULL");
  gtq_status st = gtq_decode_rotate_queries(plan, layer, cache, q, max_len, softmax_scale, chunk, workspace,
                                            ws_bytes, hip_stream);
  if (st != GTQ_OK) return st;
  st = gtq_decode_attn_partials(plan, layer, cache, seq_len, max_len, chunk, logits, workspace, ws_bytes,
                                hip_stream);
  if (st != GTQ_OK) return st;
  return gtq_decode_attn_merge(plan, layer, cache, seq_len, max_len, chunk, out, workspace, ws_bytes,
                               hip_stream);
}

gtq_status gtq_decode_attn_static(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const float* q, const int32_t* seq_len, int64_t max_len, float softmax_scale,
                                  int32_t chunk, float* out, float* logits, void* hip_stream) {
  const char* fn = "gtq_decode_attn_static";
  gtq_status st;
  if (!check_device_plan(plan, fn, &st)) return st;
  if (!cache) return fail(GTQ_EINVAL, std::string(fn) + ": cache is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(GTQ_EINVAL, std::string(fn) + ": the plan's device must be the current device");
  AttnLaunch L;
  if (!decode_shape(plan, cache->batch, max_len, chunk, &L, &st, fn)) return st;
  const size_t need = decode_ws_bytes(L.n_tiles, L.sk_G, L.qb_bytes);
  if (need > kScratchBytes)
    return fail(GTQ_ECAPACITY, std::string(fn) + ": needs " + std::to_string(need) +
                                   " bytes of workspace, more than the static scratch (" +
                                   std::to_string(kScratchBytes) + ")");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ws = (dev >= 0 && dev < kMaxScratchDevices) ? g_scratch_ptr[dev] : nullptr;
  }
  if (!ws) return fail(GTQ_EINVAL, std::string(fn) + ": no scratch address for this device");
  return gtq_decode_attn(plan, layer, cache, q, seq_len, max_len, softmax_scale, chunk, out, logits, ws,
                         kScratchBytes, hip_stream);
}

gtq_status gtq_decode_prepare(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                              const float* k_new, const float* v_new, const float* q, const int32_t* seq_len,
                              int64_t max_len, float softmax_scale, int32_t chunk, void* workspace,
                              size_t ws_bytes, void* hip_stream) {
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L, "gtq_decode_prepare");
  if (st != GTQ_OK) return st;
  if (!k_new || !v_new || !q || !seq_len) return fail(GTQ_EINVAL, "gtq_decode_prepare: NULL pointer");
  if (!isfinite(softmax_scale)) return fail(GTQ_EINVAL, "gtq_decode_prepare: softmax_scale not finite");
  AppendArgs ap{};
  fill_append_args(plan, layer, cache, k_new, v_new, ap);
  ap.step_len = seq_len;
  ap.n_tok = cache->batch;
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.prefill = 0;
  aa.max_len = (int32_t)max_len;
  aa.q = q;
  aa.qscale = softmax_scale * LOG2E_F;
  const int roles = append_roles((int64_t)cache->batch * plan->n_kv);
  const int n_app = cache->batch * plan->n_kv * roles;
  if (roles == 1 && L.tiles_per_kv == 1 && !aa.qjl)  // (then n_app == L.n_tiles)
    hipLaunchKernelGGL(decode_prep_pair_kernel, dim3((unsigned)L.n_tiles), dim3(1024), 0, (hipStream_t)hip_stream,
                       ap, aa);
  else
    hipLaunchKernelGGL(decode_prep_kernel, dim3((unsigned)(n_app + L.n_tiles)), dim3(1024), 0,
                       (hipStream_t)hip_stream, ap, aa, n_app, roles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq_decode_prepare: launch");
  return ok();
}

gtq_status gtq_decode_step(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                           const float* k_new, const float* v_new, const float* q, const int32_t* seq_len,
                           int64_t max_len, float softmax_scale, int32_t chunk, float* out, void* workspace,
                           size_t ws_bytes, void* hip_stream) {
  if (!out) return fail(GTQ_EINVAL, "gtq_decode_step: out is NULL");
  gtq_status st = gtq_decode_prepare(plan, layer, cache, k_new, v_new, q, seq_len, max_len, softmax_scale, chunk,
                                     workspace, ws_bytes, hip_stream);
  if (st != GTQ_OK) return st;
  st = gtq_decode_attn_partials(plan, layer, cache, seq_len, max_len, chunk, nullptr, workspace, ws_bytes,
                                hip_stream);
  if (st != GTQ_OK) return st;
  return gtq_decode_attn_merge(plan, layer, cache, seq_len, max_len, chunk, out, workspace, ws_bytes, hip_stream);
}

static bool prefill_shape(const gtq_plan* p, int64_t pos0, int64_t n_tok, int32_t chunk,
                          AttnLaunch* L, gtq_status* st, const char* fn) {
  if (pos0 < 0 || n_tok < 1) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": need pos0 >= 0 and n_tok >= 1");
    return false;
  }
  if (pos0 + n_tok > INT32_MAX || n_tok * (int64_t)p->n_q > INT32_MAX) {
    *st = fail(GTQ_EUNSUPPORTED, std::string(fn) + ": sizes too large");
    return false;
  }
  if (chunk < 0 || chunk % kBlk) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": chunk must be 0 or a positive multiple of 32");
    return false;
  }
  const int g = p->n_q / p->n_kv;
  const int64_t total = pos0 + n_tok;
  L->rows = n_tok * p->n_q;
  // prefill: tiles of 16 query rows (a KV head's rows are many), merged in tiles of 8
  L->rt = 16;
  L->tiles_per_kv = (int)((n_tok * g + 15) / 16);
  L->n_tiles = p->n_kv * L->tiles_per_kv;
  L->merge_tiles_per_kv = (int)((n_tok * g + 7) / 8);
  L->merge_n_tiles = p->n_kv * L->merge_tiles_per_kv;
  L->qb_bytes = attn_qb_bytes(L->n_tiles, L->rt);
  L->chunk = chunk ? chunk : auto_chunk(total, L->n_tiles, kBlk * kWaves);
  L->n_chunks = (int)((total + L->chunk - 1) / L->chunk);
  if (L->n_chunks > kMaxChunks) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": chunk too small (more than 256 splits per sequence)");
    return false;
  }
  return true;
}

gtq_status gtq_prefill_workspace_bytes(const gtq_plan* plan, int64_t pos0, int64_t n_tok,
                                       int32_t chunk, size_t* out) {
  if (!plan || !out) return fail(GTQ_EINVAL, "gtq_prefill_workspace_bytes: NULL pointer");
  AttnLaunch L;
  gtq_status st;
  if (!prefill_shape(plan, pos0, n_tok, chunk, &L, &st, "gtq_prefill_workspace_bytes")) return st;
  *out = attn_ws_bytes(L.rows, L.n_chunks, L.qb_bytes);
  return ok();
}

gtq_status gtq_prefill_attn(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                            const float* q, int32_t seq, int64_t pos0, int64_t n_tok,
                            float softmax_scale, int32_t chunk, float* out, void* workspace,
                            size_t ws_bytes, void* hip_stream) {
  gtq_status st;
  if (!check_device_plan(plan, "gtq_prefill_attn", &st)) return st;
  if (!check_cache(plan, cache, "gtq_prefill_attn", &st)) return st;
  if (layer < 0 || layer >= plan->n_layers) return fail(GTQ_EINVAL, "gtq_prefill_attn: layer out of range");
  if (seq < 0 || seq >= cache->batch) return fail(GTQ_EINVAL, "gtq_prefill_attn: seq out of range");
  if (!q || !out || !workspace) return fail(GTQ_EINVAL, "gtq_prefill_attn: NULL pointer");
  if (!isfinite(softmax_scale)) return fail(GTQ_EINVAL, "gtq_prefill_attn: softmax_scale not finite");
  if (plan->flags & GTQ_PLAN_QJL) return fail(GTQ_EUNSUPPORTED, "gtq_prefill_attn: QJL plans are decode only");
  AttnLaunch L;
  if (!prefill_shape(plan, pos0, n_tok, chunk, &L, &st, "gtq_prefill_attn")) return st;
  if (pos0 + n_tok > cache->capacity) return fail(GTQ_ECAPACITY, "gtq_prefill_attn: pos0 + n_tok > capacity");
  if (ws_bytes < attn_ws_bytes(L.rows, L.n_chunks, L.qb_bytes))
    return fail(GTQ_ECAPACITY, "gtq_prefill_attn: workspace too small");
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.logits = nullptr;
  aa.prefill = 1;
  aa.seq = seq;
  aa.pos0 = pos0;
  aa.n_tok = (int32_t)n_tok;
  aa.max_len = (int32_t)(pos0 + n_tok);
  hipStream_t s = (hipStream_t)hip_stream;
  st = launch_qrot(aa, L, q, softmax_scale, s);
  if (st != GTQ_OK) return st;
  st = launch_partials(plan, layer, aa, L, s);
  if (st != GTQ_OK) return st;
  return launch_merge(plan, layer, L, nullptr, pos0, 1, (int)(pos0 + n_tok), out, workspace, s);
}

static bool check_window(const gtq_plan* plan, int32_t layer, const gtq_window_view* w, int32_t batch,
                         const char* fn, gtq_status* st) {
  if (!w || !w->k_sink || !w->v_sink || !w->k_recent || !w->v_recent) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": window view or one of its buffers is NULL");
    return false;
  }
  if (w->n_sink < 0 || w->n_sink > 256 || w->n_recent < 0 || w->n_recent > 8192 || w->n_recent % kBlk) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": n_sink in [0, 256], n_recent a multiple of 32 in [0, 8192]");
    return false;
  }
  if (w->batch != batch) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": window batch differs from the cache's");
    return false;
  }
  if (layer < 0 || layer >= plan->n_layers) {
    *st = fail(GTQ_EINVAL, std::string(fn) + ": layer out of range");
    return false;
  }
  return true;
}

static int sink_slots_of(const gtq_window_view* w) { return (w->n_sink + kBlk - 1) / kBlk * kBlk; }

gtq_status gtq_window_append(const gtq_plan* plan, int32_t layer, const gtq_window_view* window,
                             const float* k, const float* v, const int32_t* seq_idx, const int64_t* pos,
                             int64_t n_tok, void* hip_stream) {
  gtq_status st;
  if (!check_device_plan(plan, "gtq_window_append", &st)) return st;
  if (!window) return fail(GTQ_EINVAL, "gtq_window_append: window view is NULL");
  if (!check_window(plan, layer, window, window->batch, "gtq_window_append", &st)) return st;
  if (window->batch < 1) return fail(GTQ_EINVAL, "gtq_window_append: batch < 1");
  if (n_tok < 0) return fail(GTQ_EINVAL, "gtq_window_append: n_tok < 0");
  if (n_tok == 0) return ok();
  if (!k || !v || !seq_idx || !pos) return fail(GTQ_EINVAL, "gtq_window_append: NULL pointer");
  if (n_tok > 0x7FFFFFFF) return fail(GTQ_EUNSUPPORTED, "gtq_window_append: too many tokens");
  WindowAppendArgs wa{window->k_sink, window->v_sink, window->k_recent, window->v_recent, k, v, seq_idx, pos,
                      plan->d_overflow, window->batch, plan->n_kv, window->n_sink, sink_slots_of(window),
                      window->n_recent};
  hipLaunchKernelGGL(window_append_kernel, dim3((unsigned)n_tok, plan->n_kv), dim3(kD), 0, (hipStream_t)hip_stream,
                     wa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq_window_append: launch");
  return ok();
}

gtq_status gtq_decode_window_workspace_bytes(const gtq_plan* plan, int32_t batch, int64_t max_len,
                                             int32_t chunk, size_t* out) {
  if (!plan || !out) return fail(GTQ_EINVAL, "gtq_decode_window_workspace_bytes: NULL pointer");
  if (batch < 1) return fail(GTQ_EINVAL, "gtq_decode_window_workspace_bytes: batch < 1");
  AttnLaunch L;
  gtq_status st;
  if (!decode_shape(plan, batch, max_len, chunk, &L, &st, "gtq_decode_window_workspace_bytes", 1)) return st;
  *out = decode_ws_bytes(L.n_tiles, L.sk_G, L.qb_bytes);
  return ok();
}

gtq_status gtq_decode_attn_window(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const gtq_window_view* window, const float* q, const int32_t* seq_len,
                                  int64_t max_len, float softmax_scale, int32_t chunk, float* out,
                                  float* logits, void* workspace, size_t ws_bytes, void* hip_stream) {
  const char* fn = "gtq_decode_attn_window";
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L, fn, 1);
  if (st != GTQ_OK) return st;
  if (!check_window(plan, layer, window, cache->batch, fn, &st)) return st;
  if (!q || !seq_len || !out) return fail(GTQ_EINVAL, "gtq_decode_attn_window: NULL pointer");
  if (!isfinite(softmax_scale)) return fail(GTQ_EINVAL, "gtq_decode_attn_window: softmax_scale not finite");
  hipStream_t stream = (hipStream_t)hip_stream;
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.prefill = 0;
  aa.max_len = (int32_t)max_len;
  aa.q = q;
  aa.qscale = softmax_scale * LOG2E_F;
  aa.logits = logits;
  aa.logits_ld = max_len;
  aa.seq_len = seq_len;
  aa.win = 1;
  aa.wk_sink = window->k_sink;
  aa.wv_sink = window->v_sink;
  aa.wk_rec = window->k_recent;
  aa.wv_rec = window->v_recent;
  aa.n_sink = window->n_sink;
  aa.sink_slots = sink_slots_of(window);
  aa.n_recent = window->n_recent;
  hipLaunchKernelGGL(attn_qrot_window_kernel, dim3((unsigned)(2 * L.n_tiles)), dim3(64 * kQrotWaves), 0, stream, aa,
                     L.n_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq_decode_attn_window: launch");
  st = launch_partials(plan, layer, aa, L, stream);
  if (st != GTQ_OK) return st;
  return launch_merge(plan, layer, L, seq_len, 0, 0, (int)max_len, out, workspace, stream, window);
}

gtq_status gtq_decode_step_window(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const gtq_window_view* window, const float* k_new, const float* v_new,
                                  const float* q, const int32_t* seq_len, int64_t max_len, float softmax_scale,
                                  int32_t chunk, float* out, void* workspace, size_t ws_bytes, void* hip_stream) {
  const char* fn = "gtq_decode_step_window";
  AttnLaunch L;
  gtq_status st = decode_check(plan, layer, cache, max_len, chunk, ws_bytes, workspace, &L, fn, 1);
  if (st != GTQ_OK) return st;
  if (!check_window(plan, layer, window, cache->batch, fn, &st)) return st;
  if (!k_new || !v_new || !q || !seq_len || !out) return fail(GTQ_EINVAL, "gtq_decode_step_window: NULL pointer");
  if (!isfinite(softmax_scale)) return fail(GTQ_EINVAL, "gtq_decode_step_window: softmax_scale not finite");
  if (L.tiles_per_kv != 1)
    return fail(GTQ_EUNSUPPORTED, "gtq_decode_step_window: more than 8 query heads per KV head (use the "
                                  "separate appends and gtq_decode_attn_window)");
  hipStream_t stream = (hipStream_t)hip_stream;
  AppendArgs ap{};
  fill_append_args(plan, layer, cache, k_new, v_new, ap);
  ap.step_len = seq_len;
  ap.n_tok = cache->batch;
  AttnArgs aa{};
  fill_attn_args(plan, layer, cache, aa, L, workspace);
  aa.prefill = 0;
  aa.max_len = (int32_t)max_len;
  aa.q = q;
  aa.qscale = softmax_scale * LOG2E_F;
  aa.seq_len = seq_len;
  aa.win = 1;
  aa.wk_sink = window->k_sink;
  aa.wv_sink = window->v_sink;
  aa.wk_rec = window->k_recent;
  aa.wv_rec = window->v_recent;
  aa.n_sink = window->n_sink;
  aa.sink_slots = sink_slots_of(window);
  aa.n_recent = window->n_recent;
  WindowAppendArgs wa{window->k_sink, window->v_sink, window->k_recent, window->v_recent, k_new, v_new, nullptr,
                      nullptr, plan->d_overflow, window->batch, plan->n_kv, window->n_sink, sink_slots_of(window),
                      window->n_recent};
  const int roles = append_roles((int64_t)cache->batch * plan->n_kv);
  const int n_app = cache->batch * plan->n_kv * roles;
  hipLaunchKernelGGL(decode_prep_window_kernel, dim3((unsigned)(n_app + 2 * L.n_tiles)), dim3(1024), 0, stream, ap,
                     aa, wa, n_app, roles, L.n_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "gtq_decode_step_window: launch");
  st = launch_partials(plan, layer, aa, L, stream);
  if (st != GTQ_OK) return st;
  return launch_merge(plan, layer, L, seq_len, 0, 0, (int)max_len, out, workspace, stream, window);
}

}  // extern "C"
