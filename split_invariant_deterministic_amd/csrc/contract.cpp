// Serialized execution contract and its identity digests (host only).
//
// IsoExec blog, "Unified execution contract": the contract lists the cases a
// token's logprob is computed under, a composition that maps each region to
// an implementation and the constants pinned for it, claims (the parallel
// sizes proven invariant), and three SHA-256 identities of the serialized
// contract. The semantic digest identifies the logical model, the
// numerical_policy digest every choice that can move a bit, and the
// deployment digest the settings proven not to move bits, which two
// runtimes need not share. Peers exchange digests and refuse to run when the
// semantic or numerical_policy digests differ.
//
// The text is compact JSON with a fixed key order, integers and ASCII
// strings only (floats are written as their IEEE-754 bit patterns), so that
// one contract has exactly one byte sequence. Entries are sorted by region.
//   semantic digest          = SHA-256 of the "semantic" value
//   numerical_policy digest  = SHA-256 of {"cases":..,"composition":..,"claims":..}
//   deployment digest        = SHA-256 of the "deployment" value
//
// SHA-256 follows FIPS 180-4; its round constants and initial hash value are
// derived here from the primes (fractional bits of cube and square roots)
// with exact integer arithmetic rather than written out.
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/inv.h"

namespace {

// ------------------------------------------------------------------ SHA-256

typedef unsigned __int128 u128;

struct ShaTables {
  uint32_t k[64];
  uint32_t h0[8];
  ShaTables() {
    uint32_t primes[64];
    int n = 0;
    for (uint32_t v = 2; n < 64; ++v) {
      bool prime = true;
      for (uint32_t d = 2; d * d <= v; ++d)
        if (v % d == 0) {
          prime = false;
          break;
        }
      if (prime) primes[n++] = v;
    }
    // floor(cbrt(p) * 2^32) = icbrt(p * 2^96); the low 32 bits are the fraction
    for (int i = 0; i < 64; ++i) {
      const u128 x = (u128)primes[i] << 96;
      uint64_t lo = 0, hi = (uint64_t)1 << 37;
      while (lo < hi) {
        const uint64_t mid = lo + (hi - lo + 1) / 2;
        if ((u128)mid * mid * mid <= x) lo = mid;
        else hi = mid - 1;
      }
      k[i] = (uint32_t)lo;
    }
    // floor(sqrt(p) * 2^32) = isqrt(p * 2^64)
    for (int i = 0; i < 8; ++i) {
      const u128 x = (u128)primes[i] << 64;
      uint64_t lo = 0, hi = (uint64_t)1 << 36;
      while (lo < hi) {
        const uint64_t mid = lo + (hi - lo + 1) / 2;
        if ((u128)mid * mid <= x) lo = mid;
        else hi = mid - 1;
      }
      h0[i] = (uint32_t)lo;
    }
  }
};

const ShaTables& sha_tables() {
  static const ShaTables t;  // thread-safe one-time initialisation
  return t;
}

inline uint32_t rotr(uint32_t x, int s) { return (x >> s) | (x << (32 - s)); }

void sha_block(uint32_t h[8], const uint8_t* p, const uint32_t* k) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)p[4 * t] << 24 | (uint32_t)p[4 * t + 1] << 16 | (uint32_t)p[4 * t + 2] << 8 | p[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + k[t] + w[t];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    hh = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h[0] += a;
  h[1] += b;
  h[2] += c;
  h[3] += d;
  h[4] += e;
  h[5] += f;
  h[6] += g;
  h[7] += hh;
}

void sha256(const uint8_t* data, size_t n, uint8_t out[32]) {
  const ShaTables& T = sha_tables();
  uint32_t h[8];
  std::memcpy(h, T.h0, sizeof(h));
  size_t i = 0;
  for (; i + 64 <= n; i += 64) sha_block(h, data + i, T.k);
  // padding: 0x80, zeros, then the bit length as a 64-bit big-endian integer
  uint8_t tail[128] = {0};
  const size_t rem = n - i;
  if (rem) std::memcpy(tail, data + i, rem);  // data may be NULL when n == 0
  tail[rem] = 0x80;
  const size_t tl = rem + 1 + 8 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)n * 8u;
  for (int b = 0; b < 8; ++b) tail[tl - 1 - b] = (uint8_t)(bits >> (8 * b));
  for (size_t o = 0; o < tl; o += 64) sha_block(h, tail + o, T.k);
  for (int j = 0; j < 8; ++j) {
    out[4 * j] = (uint8_t)(h[j] >> 24);
    out[4 * j + 1] = (uint8_t)(h[j] >> 16);
    out[4 * j + 2] = (uint8_t)(h[j] >> 8);
    out[4 * j + 3] = (uint8_t)h[j];
  }
}

std::string hex(const uint8_t* d, size_t n) {
  static const char* digits = "0123456789abcdef";
  std::string s;
  for (size_t i = 0; i < n; ++i) {
    s += digits[d[i] >> 4];
    s += digits[d[i] & 15];
  }
  return s;
}

// ------------------------------------------------------------------ regions

struct RegionInfo {
  int region;
  const char* name;
  int op;            // inv_op used to validate the region's contract
  const char* impl;  // implementation id in this library
  uint32_t version;
};

const RegionInfo kRegions[] = {
    {INV_REGION_NORM, "norms.rms", INV_OP_RMSNORM, "rmsnorm_row_wave", 1},
    {INV_REGION_LINEAR, "linear", INV_OP_GEMM, "k_leaf_mfma_tree", 1},
    {INV_REGION_LM_HEAD, "lm_head", INV_OP_GEMM, "k_leaf_mfma_tree", 1},
    {INV_REGION_LOGPROB, "logprob", INV_OP_LOGPROB, "vocab_chunk_tree", 1},
    {INV_REGION_ATTENTION, "attention", INV_OP_DECODE_ATTN, "split_kv_online_softmax", 1},
    {INV_REGION_MOE_ROUTE, "moe.route", INV_OP_MOE_ROUTE, "topk_softmax_lower_id_ties", 1},
    {INV_REGION_MOE_EXPERTS, "moe.experts", INV_OP_MOE_GEMM, "grouped_k_leaf_mfma_tree", 1},
    {INV_REGION_MOE_COMBINE, "moe.combine", INV_OP_MOE_COMBINE, "expert_id_leaf_tree", 1},
    {INV_REGION_LMHEAD_LOGPROB, "lm_head_logprob", INV_OP_LMHEAD_LOGPROB, "k_leaf_mfma_tree_block16_epilogue", 1},
    {INV_REGION_GDN, "gdn.core", INV_OP_GDN_PREFILL, "cpr_boundary_closed_form_recurrent_scan", 1},
};

const RegionInfo* region_info(int region) {
  for (const RegionInfo& r : kRegions)
    if (r.region == region) return &r;
  return nullptr;
}

const char* dtype_name(int d) { return d == INV_BF16 ? "bf16" : "fp32"; }
const char* tree_name(int t) { return t == INV_TREE_LEFT_FOLD ? "left_fold" : "balanced"; }

std::string u(uint64_t v) { return std::to_string(v); }
std::string q(const char* s) { return std::string("\"") + s + "\""; }

const char* const kCases = "[\"trainer_fwd\",\"trainer_fwd_no_autograd\",\"engine_prefill\",\"engine_decode\"]";

// powers of two dividing n: the rank counts whose blocks are subtrees
std::string proven(uint32_t n) {
  std::string s = "[";
  for (uint32_t r = 1; r <= n; r *= 2)
    if (n % r == 0) s += (s.size() > 1 ? "," : "") + u(r);
  return s + "]";
}

std::string constants(const RegionInfo& r, const inv_contract& c) {
  const std::string acc = ",\"accum_dtype\":" + q(dtype_name(c.accum_dtype));
  switch (r.region) {
    case INV_REGION_NORM:
      return "{\"sum\":\"fp32 squares, fixed wave butterfly\"" + acc + ",\"out_dtype\":\"bf16\"}";
    case INV_REGION_LINEAR:
    case INV_REGION_LM_HEAD:
    case INV_REGION_MOE_EXPERTS:
      return "{\"leaves\":" + u(c.leaves) + ",\"tree\":" + q(tree_name(c.tree)) + acc +
             ",\"leaf_dtype\":" + q(dtype_name(c.leaf_dtype)) + ",\"out_dtype\":" + q(dtype_name(c.out_dtype)) +
             ",\"leaf_chain\":\"v_mfma_f32_16x16x32_bf16, ascending k from +0\"}";
    case INV_REGION_LOGPROB:
      return "{\"chunks\":" + u(c.leaves) + ",\"tree\":" + q(tree_name(c.tree)) + acc +
             ",\"exp\":\"exp2 of the fp32-rounded product with log2(e)\",\"merge\":\"max-shifted (m, s)\"}";
    case INV_REGION_ATTENTION:
      return "{\"split_kv\":" + u(c.split_kv) + ",\"kv_chunk\":" + u(c.kv_chunk) + ",\"tree\":" +
             q(tree_name(c.tree)) + acc + ",\"p_operand\":\"bf16 hi + bf16 lo\",\"out_dtype\":\"bf16\"}";
    case INV_REGION_MOE_ROUTE:
      return "{\"weights\":\"fp32 softmax over the top k\",\"ties\":\"lower expert id\"}";
    case INV_REGION_LMHEAD_LOGPROB:
      return "{\"leaves\":" + u(c.leaves) + ",\"tree\":" + q(tree_name(c.tree)) + acc +
             ",\"leaf_dtype\":" + q(dtype_name(c.leaf_dtype)) + ",\"logits_dtype\":\"fp32\"" +
             ",\"leaf_chain\":\"v_mfma_f32_16x16x32_bf16, ascending k from +0\"" +
             ",\"vocab_block\":16,\"block_sum\":\"balanced over the column index\"" +
             ",\"block_merge\":\"balanced, padded with (-inf, 0) to a power of two\"}";
    case INV_REGION_GDN:
      return "{\"chunk\":" + u(c.kv_chunk) + acc + ",\"state_dtype\":\"fp32\",\"out_dtype\":" +
             q(dtype_name(c.out_dtype)) +
             ",\"boundary\":\"chunkwise closed form, unit-lower-triangular solve by forward substitution\"" +
             ",\"outputs\":\"token recurrence from the chunk's boundary state\"" +
             ",\"decode\":\"recurrence, resynchronised to the boundary state when a chunk closes\"}";
    case INV_REGION_MOE_COMBINE:
      return "{\"leaves\":" + u(c.leaves) + ",\"tree\":" + q(tree_name(c.tree)) + acc +
             ",\"leaf_order\":\"ascending expert id\",\"out_dtype\":\"bf16\"}";
  }
  return "{}";
}

struct Sections {
  std::string semantic, policy, deployment;
};

// Validates the entries and builds the three hashed sections.
inv_status build(const inv_region_contract* e, size_t n, Sections& out) {
  if (!e || n == 0 || n > sizeof(kRegions) / sizeof(kRegions[0])) return INV_E_ARG;
  const inv_region_contract* sorted[sizeof(kRegions) / sizeof(kRegions[0])];
  size_t m = 0;
  for (const RegionInfo& r : kRegions) {
    const inv_region_contract* hit = nullptr;
    for (size_t i = 0; i < n; ++i)
      if (e[i].region == r.region) {
        if (hit) return INV_E_ARG;  // a region listed twice
        hit = &e[i];
      }
    if (hit) sorted[m++] = hit;
  }
  if (m != n) return INV_E_ARG;  // an unknown region id
  for (size_t i = 0; i < m; ++i) {
    if (sorted[i]->reserved != 0) return INV_E_ARG;
    const RegionInfo& r = *region_info(sorted[i]->region);
    const inv_contract& c = sorted[i]->contract;
    const int64_t K =
        (r.op == INV_OP_GEMM || r.op == INV_OP_MOE_GEMM || r.op == INV_OP_LMHEAD_LOGPROB) ? (int64_t)c.leaves * 32 : 0;
    const inv_status s = inv_contract_check(&c, r.op, K);
    if (s != INV_OK) return s;
  }

  std::string names = "[", sem_const = "{", comp = "[", topo = "{", ranks = "{";
  for (size_t i = 0; i < m; ++i) {
    const RegionInfo& r = *region_info(sorted[i]->region);
    const inv_contract& c = sorted[i]->contract;
    const std::string sep = i ? "," : "";
    names += sep + q(r.name);
    comp += sep + "{\"region\":" + q(r.name) + ",\"cases\":" + kCases + ",\"impl\":{\"id\":" + q(r.impl) +
            ",\"version\":" + u(r.version) + ",\"arch\":\"gfx950\"},\"constants\":" + constants(r, c) + "}";
    topo += sep + q(r.name) + ":{\"proven_ranks\":" +
            (r.region == INV_REGION_MOE_EXPERTS || r.region == INV_REGION_LMHEAD_LOGPROB || r.region == INV_REGION_GDN
                 ? std::string("[1]")
                                                                                        : proven(c.leaves)) +
            "}";
    ranks += sep + q(r.name) + ":" + u(c.ranks);
    if (r.region == INV_REGION_NORM) {
      uint32_t bits;
      std::memcpy(&bits, &c.eps, 4);
      char buf[16];
      std::snprintf(buf, sizeof(buf), "0x%08x", bits);
      sem_const += std::string(sem_const.size() > 1 ? "," : "") + q(r.name) + ":{\"eps_fp32_bits\":" + q(buf) + "}";
    } else if (r.region == INV_REGION_GDN) {
      sem_const += std::string(sem_const.size() > 1 ? "," : "") + q(r.name) +
                   ":{\"head_width\":128,\"l2norm_eps_fp32_bits\":\"0x358637bd\",\"gate\":\"alpha = exp(g)\"}";
    } else if (r.region == INV_REGION_MOE_ROUTE || r.region == INV_REGION_MOE_COMBINE) {
      sem_const += std::string(sem_const.size() > 1 ? "," : "") + q(r.name) + ":{\"top_k\":" + u(c.leaves) + "}";
    }
  }
  out.semantic = "{\"regions\":" + names + "],\"constants\":" + sem_const + "}}";
  out.policy = std::string("{\"cases\":") + kCases + ",\"composition\":" + comp + "],\"claims\":{\"topology\":" +
               topo + "}}}";
  out.deployment = "{\"abi_version\":" + u(INV_ABI_VERSION) + ",\"ranks\":" + ranks +
                   "},\"workspace\":\"caller-owned, sized by inv_workspace_bytes\"}";
  return INV_OK;
}

void digest_of(const Sections& s, int kind, uint8_t out[32]) {
  const std::string& t = kind == INV_DIGEST_SEMANTIC ? s.semantic
                          : kind == INV_DIGEST_NUMERICAL_POLICY ? s.policy
                                                                : s.deployment;
  sha256(reinterpret_cast<const uint8_t*>(t.data()), t.size(), out);
}

bool valid_kind(int kind) {
  return kind == INV_DIGEST_SEMANTIC || kind == INV_DIGEST_NUMERICAL_POLICY || kind == INV_DIGEST_DEPLOYMENT;
}

}  // namespace

extern "C" {

inv_status inv_sha256(const void* data, size_t bytes, uint8_t digest[32]) {
  if ((!data && bytes) || !digest) return INV_E_ARG;
  sha256(static_cast<const uint8_t*>(data), bytes, digest);
  return INV_OK;
}

inv_status inv_contract_json(const inv_region_contract* entries, size_t n, char* buf, size_t cap, size_t* len) {
  if (!len) return INV_E_ARG;
  Sections s;
  try {
    const inv_status st = build(entries, n, s);
    if (st != INV_OK) return st;
    uint8_t d[3][32];
    for (int k = 0; k < 3; ++k) digest_of(s, k + 1, d[k]);
    // the policy section is an object whose members are spliced in unchanged
    const std::string policy_members = s.policy.substr(1, s.policy.size() - 2);
    const std::string text = "{\"ExecutionContract\":{" + policy_members + ",\"semantic\":" + s.semantic +
                             ",\"deployment\":" + s.deployment + ",\"identities\":{\"semantic\":\"" +
                             hex(d[0], 32) + "\",\"numerical_policy\":\"" + hex(d[1], 32) +
                             "\",\"deployment\":\"" + hex(d[2], 32) + "\"}}}";
    *len = text.size();
    if (!buf) return INV_OK;  // size query
    if (cap < text.size() + 1) return INV_E_ARG;
    std::memcpy(buf, text.c_str(), text.size() + 1);
    return INV_OK;
  } catch (...) {
    return INV_E_ARG;  // allocation failure; nothing written
  }
}

inv_status inv_contract_digest(const inv_region_contract* entries, size_t n, int kind, uint8_t digest[32]) {
  if (!digest || !valid_kind(kind)) return INV_E_ARG;
  Sections s;
  try {
    const inv_status st = build(entries, n, s);
    if (st != INV_OK) return st;
    digest_of(s, kind, digest);
    return INV_OK;
  } catch (...) {
    return INV_E_ARG;
  }
}

inv_status inv_contract_verify(const inv_region_contract* entries, size_t n, int kind,
                               const uint8_t expected[32]) {
  if (!expected) return INV_E_ARG;
  uint8_t d[32];
  const inv_status st = inv_contract_digest(entries, n, kind, d);
  if (st != INV_OK) return st;
  return std::memcmp(d, expected, 32) == 0 ? INV_OK : INV_E_CONTRACT;
}

}  // extern "C"
