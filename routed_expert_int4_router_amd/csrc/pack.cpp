// Host-side record geometry, the affine group quantiser and the packer.
//
// The pages describe the container only as fixed-stride expert blobs, one read
// of the record bytes at base + index * stride (paotong.dev commentary,
// paragraph on the fetch path), holding MLX-style int4/int8 group-quantised
// weights with 64-bit offsets (cheshm.ai news article, paragraph on the code
// base). The record layout and the min/max grid are documented in moe.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "common.h"

namespace moe {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }
void clear_error() { g_err.clear(); }
moe_status fail(moe_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

static bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

std::string check_config(const moe_config* c) {
  if (!c) return "config is NULL";
  if (c->bits != 4 && c->bits != 8) return "bits must be 4 or 8";
  if (c->group != 64) return "group must be 64";
  if (!pow2_in(c->hidden, 64, 4096)) return "hidden must be a power of two in [64, 4096]";
  if (!pow2_in(c->inter, 64, 4096)) return "inter must be a power of two in [64, 4096]";
  if (c->shared_inter != c->inter) return "shared_inter must equal inter";
  if (c->hidden * c->bits > 16384 || c->inter * c->bits > 16384)
    return "a code row may hold at most 2048 bytes (hidden*bits and inter*bits <= 16384)";
  if (c->n_experts < 1 || c->n_experts > 1024) return "n_experts must be in [1, 1024]";
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return "top_k must be in [1, min(n_experts, 16)]";
  if (c->n_layers < 1 || c->n_layers > 4096) return "n_layers must be in [1, 4096]";
  if ((c->top_k + 1) * c->inter > 15360) return "(top_k + 1) * inter must be <= 15360";
  if (c->norm_topk != 0 && c->norm_topk != 1) return "norm_topk must be 0 or 1";
  return "";
}

size_t record_bytes(const moe_config& c, int inter) {
  size_t hi = (size_t)c.hidden * (size_t)inter;
  return 3 * hi * (size_t)c.bits / 8 + 3 * (hi / 64) * 4;
}

size_t record_stride(const moe_config& c, int inter) {
  size_t n = record_bytes(c, inter);
  return (n + 4095) / 4096 * 4096;
}

RecordLayout record_layout(const moe_config& c, int inter) {
  size_t H = c.hidden, I = inter;
  size_t cgu = I * H * c.bits / 8, cd = H * I * c.bits / 8;
  size_t sgu = I * (H / 64) * 4, sd = H * (I / 64) * 4;
  RecordLayout r;
  r.gate_codes = 0;
  r.up_codes = cgu;
  r.down_codes = 2 * cgu;
  r.gate_sc = 2 * cgu + cd;
  r.up_sc = r.gate_sc + sgu;
  r.down_sc = r.up_sc + sgu;
  r.end = r.down_sc + sd;
  return r;
}

uint16_t f32_to_f16_rne(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds past 65504
  if (ax < 0x38800000u) {                                     // below 2^-14: fp16 subnormal grid 2^-24
    if (ax < 0x33000000u) return (uint16_t)sign;              // below 2^-25 rounds to zero
    uint32_t e = ax >> 23;
    uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    int shift = 126 - (int)e;  // 14..24
    uint32_t m = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (m & 1u))) m++;
    return (uint16_t)(sign | m);
  }
  uint32_t e = (ax >> 23) - 127u + 15u;
  uint32_t mant = ax & 0x7FFFFFu;
  uint32_t h = (e << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  float v;
  if (e == 0) {
    v = std::ldexp((float)m, -24);
  } else if (e == 31) {
    v = m ? std::nanf("") : INFINITY;
  } else {
    v = std::ldexp((float)(m | 0x400u), (int)e - 25);
  }
  uint32_t bits;
  std::memcpy(&bits, &v, 4);
  bits |= sign;
  std::memcpy(&v, &bits, 4);
  return v;
}

// Quantise one row [K] into codes (one byte per element) and (s,c) fp16 pairs.
// Returns false on a non-finite weight or an fp16 overflow of s or c.
static bool quantize_row(const float* w, int K, int bits, uint8_t* q, uint16_t* sc) {
  const float qmax = (float)((1 << bits) - 1);
  for (int g = 0; g < K / 64; ++g) {
    const float* wg = w + g * 64;
    float lo = wg[0], hi = wg[0];
    for (int i = 0; i < 64; ++i) {
      if (!std::isfinite(wg[i])) return false;
      lo = std::min(lo, wg[i]);
      hi = std::max(hi, wg[i]);
    }
    lo = lo + 0.0f;  // a -0 minimum is stored as +0
    volatile float range = hi - lo;
    volatile float s32 = range / qmax;
    uint16_t sh = f32_to_f16_rne(s32), ch = f32_to_f16_rne(lo);
    if ((sh & 0x7C00u) == 0x7C00u || (ch & 0x7C00u) == 0x7C00u) return false;
    sc[2 * g] = sh;
    sc[2 * g + 1] = ch;
    float sf = f16_to_f32(sh), cf = f16_to_f32(ch);
    for (int i = 0; i < 64; ++i) {
      if (sf == 0.0f) {
        q[g * 64 + i] = 0;
        continue;
      }
      volatile float d = wg[i] - cf;
      volatile float t = d / sf;
      float r = std::nearbyint((float)t);
      r = std::min(std::max(r, 0.0f), qmax);
      q[g * 64 + i] = (uint8_t)r;
    }
  }
  return true;
}

static void encode_row(const uint8_t* q, int K, int bits, uint8_t* dst) {
  if (bits == 8) {
    std::memcpy(dst, q, (size_t)K);
    return;
  }
  for (int i = 0; i < K / 2; ++i) dst[i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
}

// Pack one matrix [N][K] into its codes region and sc region: row-major codes
// and (s, c) pairs [N][K/64][2] (gate, up).
static bool pack_matrix(const float* w, int N, int K, int bits, uint8_t* codes, uint16_t* sc) {
  std::vector<uint8_t> q((size_t)K);
  size_t row_bytes = (size_t)K * bits / 8;
  for (int n = 0; n < N; ++n) {
    if (!quantize_row(w + (size_t)n * K, K, bits, q.data(), sc + (size_t)n * (K / 64) * 2)) return false;
    encode_row(q.data(), K, bits, codes + (size_t)n * row_bytes);
  }
  return true;
}

// The down matrix [N = H][K = I]: codes in 16-byte tiles [K*bits/128][N][16]
// (tile t of every row before tile t+1 of any row) and (s, c) pairs
// group-major [K/64][N][2].
static bool pack_matrix_tiled(const float* w, int N, int K, int bits, uint8_t* codes, uint16_t* sc) {
  std::vector<uint8_t> q((size_t)K), row((size_t)K * bits / 8);
  std::vector<uint16_t> sr((size_t)(K / 64) * 2);
  const size_t tiles = (size_t)K * bits / 128;
  const int G = K / 64;
  for (int n = 0; n < N; ++n) {
    if (!quantize_row(w + (size_t)n * K, K, bits, q.data(), sr.data())) return false;
    encode_row(q.data(), K, bits, row.data());
    for (size_t t = 0; t < tiles; ++t) std::memcpy(codes + (t * N + n) * 16, row.data() + t * 16, 16);
    for (int g = 0; g < G; ++g) {
      sc[((size_t)g * N + n) * 2] = sr[(size_t)2 * g];
      sc[((size_t)g * N + n) * 2 + 1] = sr[(size_t)2 * g + 1];
    }
  }
  return true;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_expert_bytes(const moe_config* cfg, int32_t inter) {
  if (!check_config(cfg).empty() || (inter != cfg->inter && inter != cfg->shared_inter)) return 0;
  return record_bytes(*cfg, inter);
}

size_t moe_expert_stride(const moe_config* cfg, int32_t inter) {
  if (!check_config(cfg).empty() || (inter != cfg->inter && inter != cfg->shared_inter)) return 0;
  return record_stride(*cfg, inter);
}

uint64_t moe_blob_offset(uint64_t base, uint64_t gid, uint64_t stride) { return base + gid * stride; }

moe_status moe_pack(const moe_config* cfg, int32_t inter, const float* w_gate, const float* w_up,
                    const float* w_down, int64_t n, void* dst, size_t dst_bytes) {
  clear_error();
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(MOE_EINVAL, "moe_pack: " + why);
  if (inter != cfg->inter && inter != cfg->shared_inter) return fail(MOE_EINVAL, "moe_pack: inter must be inter or shared_inter");
  if (n < 0) return fail(MOE_EINVAL, "moe_pack: n < 0");
  if (n == 0) return MOE_OK;
  if (!w_gate || !w_up || !w_down || !dst) return fail(MOE_EINVAL, "moe_pack: NULL pointer");
  const size_t stride = record_stride(*cfg, inter);
  if (dst_bytes / stride < (size_t)n) return fail(MOE_EINVAL, "moe_pack: dst_bytes < n * stride");
  const RecordLayout lay = record_layout(*cfg, inter);
  const int H = cfg->hidden, I = inter, bits = cfg->bits;
  const size_t gu_elems = (size_t)I * H, d_elems = (size_t)H * I;
  uint8_t* out = static_cast<uint8_t*>(dst);

  std::atomic<int64_t> next{0};
  std::atomic<int64_t> bad{-1};
  auto worker = [&]() {
    for (;;) {
      int64_t e = next.fetch_add(1);
      if (e >= n || bad.load() >= 0) return;
      uint8_t* rec = out + (size_t)e * stride;
      bool ok = pack_matrix(w_gate + (size_t)e * gu_elems, I, H, bits, rec + lay.gate_codes,
                            reinterpret_cast<uint16_t*>(rec + lay.gate_sc)) &&
                pack_matrix(w_up + (size_t)e * gu_elems, I, H, bits, rec + lay.up_codes,
                            reinterpret_cast<uint16_t*>(rec + lay.up_sc)) &&
                pack_matrix_tiled(w_down + (size_t)e * d_elems, H, I, bits, rec + lay.down_codes,
                                  reinterpret_cast<uint16_t*>(rec + lay.down_sc));
      if (!ok) {
        int64_t expect = -1;
        bad.compare_exchange_strong(expect, e);
        return;
      }
      std::memset(rec + lay.end, 0, stride - lay.end);
    }
  };
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int nthreads = (int)std::min<int64_t>(n, std::min(16u, hw));
  std::vector<std::thread> pool;
  for (int i = 1; i < nthreads; ++i) pool.emplace_back(worker);
  worker();
  for (auto& t : pool) t.join();
  if (bad.load() >= 0)
    return fail(MOE_EINVAL, "moe_pack: expert " + std::to_string(bad.load()) +
                                " has a non-finite weight or a group scale/bias that overflows fp16");
  return MOE_OK;
}

moe_status moe_unpack(const moe_config* cfg, int32_t inter, const void* record, uint8_t* q_out, uint16_t* sc_out) {
  clear_error();
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(MOE_EINVAL, "moe_unpack: " + why);
  if (inter != cfg->inter && inter != cfg->shared_inter) return fail(MOE_EINVAL, "moe_unpack: bad inter");
  if (!record || !q_out || !sc_out) return fail(MOE_EINVAL, "moe_unpack: NULL pointer");
  const RecordLayout lay = record_layout(*cfg, inter);
  const uint8_t* rec = static_cast<const uint8_t*>(record);
  const size_t H = cfg->hidden, I = inter;
  const size_t elems = 3 * H * I;
  // codes in record order with the down tiles put back into rows
  std::vector<uint8_t> bytes(elems * cfg->bits / 8);
  std::memcpy(bytes.data(), rec, lay.down_codes);
  const size_t drow = I * cfg->bits / 8, tiles = drow / 16;
  for (size_t n = 0; n < H; ++n)
    for (size_t t = 0; t < tiles; ++t)
      std::memcpy(bytes.data() + lay.down_codes + n * drow + t * 16, rec + lay.down_codes + (t * H + n) * 16, 16);
  if (cfg->bits == 8) {
    std::memcpy(q_out, bytes.data(), elems);
  } else {
    for (size_t i = 0; i < elems / 2; ++i) {
      q_out[2 * i] = bytes[i] & 0x0F;
      q_out[2 * i + 1] = bytes[i] >> 4;
    }
  }
  // (s, c) pairs: gate and up as stored, down back to [H][I/64][2]
  std::memcpy(sc_out, rec + lay.gate_sc, lay.down_sc - lay.gate_sc);
  uint16_t* dsc = sc_out + (lay.down_sc - lay.gate_sc) / 2;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(rec + lay.down_sc);
  const size_t G = I / 64;
  for (size_t n = 0; n < H; ++n)
    for (size_t g = 0; g < G; ++g) {
      dsc[(n * G + g) * 2] = src[(g * H + n) * 2];
      dsc[(n * G + g) * 2 + 1] = src[(g * H + n) * 2 + 1];
    }
  return MOE_OK;
}

}  // extern "C"
