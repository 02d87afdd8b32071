// Internal types shared by the host code and the HIP kernels of libgtq.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "gtq.h"

namespace gtq {

constexpr int kD = GTQ_HEAD_DIM;      // head dimension
constexpr int kJ = GTQ_BLOCKS;        // RoPE blocks
constexpr int kMaxGroups = GTQ_MAX_GROUPS;
constexpr int kKB = 32;               // coordinates per MFMA K-block of the decode kernel
constexpr int kMaxKB = 8;             // sum_g ceil(d_g / 32) <= 4 + 128/32
constexpr int kKP = kKB * kMaxKB;     // padded query length (halves)
constexpr int kBlk = 32;              // tokens per decode block
constexpr int kNS = GTQ_KNORM_STRIDE;
constexpr float kRotSplitScale = 16.f;  // the split rotations hold 16 * Pi (lo parts stay normal)

// Per (layer, KV head) tables, uploaded once per plan (plain data, same layout on
// host and device).
struct DevHead {
  int32_t n_groups;
  int32_t nkb;                    // MFMA K-blocks (each inside one group)
  int32_t rate[kMaxGroups];
  int32_t dim[kMaxGroups];
  int32_t bit_off[kMaxGroups];    // group start in the key record (bits)
  int32_t pos_off[kMaxGroups];    // group start in record position order (0..127)
  int32_t kp_off[kMaxGroups];     // group start in the padded K-block order
  int32_t nkb_g[kMaxGroups];      // K-blocks of each group
  // K-blocks in slot order: first the layer's n1 leading rate-1 blocks, then its n4
  // leading rate-4 blocks, then every other block in group order (see order_kblocks)
  int32_t kb_bit[kMaxKB];         // record bit of each K-block's first coordinate
  int32_t kb_rg[kMaxKB];          // rate | group << 8 of each K-block; slots past nkb repeat slot 0
  int64_t krot_off[kMaxGroups];   // float offset of Pi_g (row-major d x d) in the pool
  int64_t vrot_off;               // float offset of Pi_V (row-major 128 x 128)
  int64_t vrot_t_off;             // float offset of Pi_V^T (row-major, i.e. Pi_V column-major)
  int64_t rsk_off;                // split K rotation: the block-diagonal 128 x 128 matrix of the
                                  // Pi_g in record position order (zeros across groups), binary16
                                  // hi then lo
  int64_t rsv_off;                // split V rotation: hi then lo, 128 x 128
  int32_t krot_floats;            // sum_g d_g^2
  int32_t v_hadamard;             // 1: Pi_V = H_128 diag(vsign) / sqrt(128) exactly (fast transform)
  int32_t mse_words;              // words of the MSE part of a key record
  int32_t qjl;                    // 1: the record goes on with the residual sketch (4 words) and gamma
  int64_t qjl_off;                // float offset of the sketch matrix S (row-major 128 x 128)
  uint8_t coord[kD];              // record position -> head coordinate
  uint8_t kp_pos[kD];             // record position -> its place in the K-block operands
                                  // (slot * 32 + coordinate within the block)
  float vsign[kD];                // the sign vector of a Hadamard Pi_V
};

constexpr int kPairTable = 340;  // (code, code) pairs of rates 1..4: 4 + 16 + 64 + 256 entries

struct DevCodebook {
  float c[5][16];   // c[b][k]: centroid k of rate b (binary16 values)
  float t[5][16];   // t[b][k]: threshold k of rate b (midpoints), k < 2^b - 1
  // decode table: entry (4^b - 4) / 3 + (k0 | k1 << b) holds the binary16 centroids
  // k0 (low half) and k1 (high half) of rate b
  uint32_t pair[kPairTable + 4];
  // byte-indexed tables of the two lowest rates: oct1[x] = the 8 binary16 centroids of
  // the eight 1-bit codes in byte x (code k at bit k; entry word j = codes 2j, 2j + 1),
  // quad2[x] = the 4 centroids of the four 2-bit codes in byte x (code k at bits 2k..)
  uint32_t oct1[256][4];
  uint32_t quad2[256][2];
};

}  // namespace gtq

struct gtq_plan {
  int32_t n_layers = 0, n_kv = 0, n_q = 0, rope_layout = 0, k_budget = 0, v_bits = 0;
  int32_t k_words = 0, flags = 0;
  std::vector<gtq::DevHead> heads;      // [L][H_kv]
  std::vector<int32_t> layer_n1, layer_n4;  // [L]: specialized rate-1 / rate-4 K-block slots
  std::vector<gtq_head_layout> layouts; // [L][H_kv]
  std::vector<float> rot;               // rotation pool
  std::vector<uint16_t> rsplit;         // rotations as binary16 (hi, lo) pairs, for the append GEMM
  gtq::DevCodebook cb{};
  // device copies (null for host-only plans)
  int device = -1;
  int n_cu = 256;                       // compute units of the device (decode partials workgroups)
  gtq::DevHead* d_heads = nullptr;
  float* d_rot = nullptr;
  uint16_t* d_rsplit = nullptr;
  gtq::DevCodebook* d_cb = nullptr;
  unsigned long long* d_overflow = nullptr;
};

namespace gtq {
gtq_status fail(gtq_status st, const std::string& msg);
gtq_status ok();
// host math shared by the host entry points
void lloyd_max(int bits, double* centroids, double* mse);
void build_head(const uint8_t* rates, int rope_layout, gtq_head_layout* lay, DevHead* dh);
void order_kblocks(DevHead* dh, int n1, int n4);
void fill_codebook(DevCodebook* cb);
gtq_status plan_build_host(const gtq_plan_desc* d, gtq_plan* p);
}  // namespace gtq
