// Host-side driver for the sanitizer build of the C-ABI layer: contract and
// shape validation of every entry point, workspace sizing, status strings,
// the contract JSON, its digests and SHA-256. Every call it makes is one
// that the library must reject, or an empty one, before any launch; each
// status is checked. Exits non-zero on the first mismatch. Built with
// -fsanitize=address,undefined so that out-of-bounds accesses, overflows
// and undefined behaviour in the host code fail the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/inv.h"

static int g_checks = 0;

#define EXPECT(call, want)                                                                           \
  do {                                                                                               \
    const int got_ = (int)(call);                                                                    \
    ++g_checks;                                                                                      \
    if (got_ != (int)(want)) {                                                                       \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
                   (int)(want));                                                                     \
      std::exit(1);                                                                                  \
    }                                                                                                \
  } while (0)

static inv_contract dflt() {
  inv_contract c;
  inv_contract_default(&c);
  return c;
}

static inv_contract with(uint32_t leaves, uint32_t ranks = 1, int out = INV_BF16, int tree = INV_TREE_BALANCED) {
  inv_contract c = dflt();
  c.leaves = leaves;
  c.ranks = ranks;
  c.out_dtype = out;
  c.tree = tree;
  return c;
}

// aligned stand-in addresses: never dereferenced (every call below fails
// validation or is empty before anything is launched)
static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t{1} << 24) + off); }

static void contracts() {
  EXPECT(inv_contract_default(nullptr), INV_E_ARG);
  inv_contract c = dflt();
  EXPECT(c.struct_size, sizeof(inv_contract));
  EXPECT(inv_contract_check(&c, INV_OP_GEMM, 4096), INV_OK);
  EXPECT(inv_contract_check(nullptr, INV_OP_GEMM, 4096), INV_E_ARG);
  EXPECT(inv_contract_check(&c, 999, 4096), INV_E_ARG);
  for (uint32_t r : {1u, 2u, 4u, 8u}) {
    inv_contract cr = with(8, r);
    EXPECT(inv_contract_check(&cr, INV_OP_GEMM, 4096), INV_OK);
  }
  for (uint32_t r : {0u, 3u, 5u, 6u, 7u, 16u}) {
    inv_contract cr = with(8, r);
    EXPECT(inv_contract_check(&cr, INV_OP_GEMM, 4096), INV_E_TOPOLOGY);
  }
  inv_contract bad = with(6);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, 6 * 64), INV_E_CONTRACT);
  bad = with(8);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, 8 * 48), INV_E_CONTRACT);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, -8), INV_E_ARG);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, 0), INV_E_CONTRACT);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, int64_t{1} << 24), INV_E_UNSUPPORTED);
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, INT64_MAX), INV_E_UNSUPPORTED);
  bad.struct_size = 4;
  EXPECT(inv_contract_check(&bad, INV_OP_GEMM, 4096), INV_E_ARG);
  bad = dflt();
  bad.abi_version = 99;
  EXPECT(inv_contract_check(&bad, INV_OP_RMSNORM, 0), INV_E_ARG);
  bad = dflt();
  bad.eps = -1.0f;
  EXPECT(inv_contract_check(&bad, INV_OP_RMSNORM, 0), INV_E_CONTRACT);
  bad = dflt();
  bad.split_kv = 12;
  EXPECT(inv_contract_check(&bad, INV_OP_DECODE_ATTN, 0), INV_E_CONTRACT);
  bad = dflt();
  bad.tree = 77;
  EXPECT(inv_contract_check(&bad, INV_OP_LOGPROB, 0), INV_E_CONTRACT);
  for (int s = -1; s < 9; ++s) {  // every string is printable and terminated
    const char* t = inv_status_string((inv_status)s);
    if (!t || std::strlen(t) == 0) std::exit(2);
  }
}

static void workspaces() {
  inv_contract c = dflt();
  EXPECT(inv_workspace_bytes(&c, INV_OP_GEMM, -1, 4, 4096), (size_t)-1);
  EXPECT(inv_workspace_bytes(&c, INV_OP_GEMM, 7, 128, 4096), 0);
  EXPECT(inv_workspace_bytes(&c, INV_OP_GEMM, 64, 128, 4096), (size_t)8 * 64 * 128 * 4);
  inv_contract c2 = with(8, 2);
  EXPECT(inv_workspace_bytes(&c2, INV_OP_GEMM, 64, 128, 4096), (size_t)2 * 64 * 128 * 4);
  EXPECT(inv_workspace_bytes(&c, INV_OP_DECODE_ATTN, 3, 32, 128), (size_t)3 * 32 * 16 * 130 * 4);
  EXPECT(inv_workspace_bytes(&c, INV_OP_LMHEAD_LOGPROB, 4, 0, 4096), (size_t)-1);
  inv_contract cf = with(8, 1, INV_FP32);
  EXPECT(inv_workspace_bytes(&cf, INV_OP_LMHEAD_LOGPROB, 4, 17, 4096), (size_t)4 * 2 * 8 + 4 * 4);
  EXPECT(inv_workspace_bytes(&cf, INV_OP_LMHEAD_LOGPROB, 4, 16 * 16384 + 1, 4096), (size_t)-1);
  EXPECT(inv_workspace_bytes(&c, INV_OP_GDN_PREFILL, 64, 0, 1), (size_t)-1);
  EXPECT(inv_workspace_bytes(&c, 12345, 1, 1, 1), (size_t)-1);
  EXPECT(inv_gdn_cache_bytes(&c, 0), (size_t)-1);
  if (inv_gdn_cache_bytes(&c, 16) == (size_t)-1) std::exit(3);
}

static void entry_points() {
  inv_contract c = dflt();
  inv_contract c3 = with(8, 3);
  inv_contract c2 = with(8, 2);
  void* f = fake();
  void* mis = fake(2);
  float* ff = static_cast<float*>(f);
  EXPECT(inv_gemm(&c3, f, f, f, 4, 4, 4096, nullptr, 0, nullptr), INV_E_TOPOLOGY);
  EXPECT(inv_gemm(&c, nullptr, nullptr, nullptr, 4, 4, 4096, nullptr, 0, nullptr), INV_E_ARG);
  EXPECT(inv_gemm(&c, f, f, f, -1, 4, 4096, nullptr, 0, nullptr), INV_E_ARG);
  EXPECT(inv_gemm(&c, f, f, f, 0, 4, 4096, nullptr, 0, nullptr), INV_OK);
  EXPECT(inv_gemm(&c, mis, f, f, 4, 4, 4096, nullptr, 0, nullptr), INV_E_ARG);
  EXPECT(inv_gemm(&c2, f, f, f, 4, 4, 4096, nullptr, 0, nullptr), INV_E_WORKSPACE);
  EXPECT(inv_gemm(&c, f, f, f, int64_t{1} << 40, 4, 4096, nullptr, 0, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_gemm_noalloc(&c3, f, f, f, 4, 4, 4096, nullptr), INV_E_TOPOLOGY);
  EXPECT(inv_gemm_noalloc(&c, f, f, f, 0, 4, 4096, nullptr), INV_OK);
  inv_contract c8r = with(8, 8);
  EXPECT(inv_gemm_noalloc(&c8r, f, f, f, 4096, 4096, 4096, nullptr), INV_E_WORKSPACE);
  EXPECT(inv_gemm_rank(&c2, f, f, ff, 4, 4, 4096, 2, nullptr), INV_E_ARG);
  EXPECT(inv_gemm_leaves(&c, f, f, ff, 4, 4, 4096, 3, 3, nullptr), INV_E_ARG);
  EXPECT(inv_gemm_leaves(&c, f, f, ff, 4, 4, 4096, 0, 9, nullptr), INV_E_ARG);
  EXPECT(inv_tree_combine(&c, ff, 3, f, 4, 4, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_tree_combine(&c, ff, 128, f, 4, 4, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_tree_combine(&c, nullptr, 4, nullptr, 0, 4, nullptr), INV_OK);
  EXPECT(inv_cast_bf16(nullptr, nullptr, -1, nullptr), INV_E_ARG);
  EXPECT(inv_cast_bf16(nullptr, nullptr, 0, nullptr), INV_OK);
  EXPECT(inv_rmsnorm(&c, f, f, f, 4, 12, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_rmsnorm(&c, f, f, f, 4, 16392, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_rmsnorm(&c, mis, f, f, 4, 4096, nullptr), INV_E_ARG);
  EXPECT(inv_rmsnorm(&c, nullptr, nullptr, nullptr, 0, 4096, nullptr), INV_OK);
  inv_contract c64 = with(64);
  EXPECT(inv_logprob(&c64, (float*)f, 10, (int32_t*)f, (float*)f, 4, 32, nullptr), INV_E_CONTRACT);
  EXPECT(inv_logprob(&c64, (float*)f, 10, (int32_t*)f, (float*)f, 4, 100, nullptr), INV_E_ARG);
  inv_contract c1024 = with(1024);
  EXPECT(inv_logprob(&c1024, (float*)f, 4096, (int32_t*)f, (float*)f, 4, 4096, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_logprob_partials(&c64, (float*)f, 4096, (int32_t*)f, (float*)f, (float*)f, 4, 4096, 8, 8, nullptr),
         INV_E_ARG);
  EXPECT(inv_logprob_combine(&c64, nullptr, nullptr, nullptr, nullptr, 4, 4096, nullptr), INV_E_ARG);
  int32_t dummy = 0;
  EXPECT(inv_decode_attn(&c, f, f, f, &dummy, 1, &dummy, &dummy, f, 1, 32, 8, 64, f, 1 << 30, nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_decode_attn(&c, f, f, f, &dummy, 1, &dummy, &dummy, f, 1, 32, 6, 128, f, 1 << 30, nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_decode_attn(&c, f, f, f, &dummy, 1, &dummy, &dummy, f, 1, 32, 8, 128, f, 16, nullptr),
         INV_E_WORKSPACE);
  EXPECT(inv_decode_attn(&c, f, f, f, &dummy, 1, &dummy, &dummy, f, 0, 32, 8, 128, nullptr, 0, nullptr), INV_OK);
  EXPECT(inv_attn_splits(&c, f, f, f, &dummy, 1, &dummy, &dummy, 1, 32, 8, 128, 4, 4, f, 1 << 30, nullptr),
         INV_E_ARG);
  EXPECT(inv_attn_combine(&c, f, 16, f, 1, 32, 128, nullptr), INV_E_WORKSPACE);
  EXPECT(inv_moe_route(&c, (float*)f, (int32_t*)f, (float*)f, 4, 300, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_moe_route(&c, (float*)f, (int32_t*)f, (float*)f, 4, 4, nullptr), INV_E_UNSUPPORTED);
  EXPECT(inv_moe_permute(&c, nullptr, nullptr, nullptr, nullptr, 4, 128, nullptr), INV_E_ARG);
  EXPECT(inv_moe_gemm(&c2, f, 4, nullptr, (int32_t*)f, f, f, 4, 2, 64, 4096, nullptr), INV_E_TOPOLOGY);
  EXPECT(inv_moe_gemm(&c, f, 4, nullptr, (int32_t*)f, f, f, 4, 2, 64, int64_t{1} << 24, nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_moe_gemm_swiglu(&c, f, 4, nullptr, (int32_t*)f, f, f, 4, 2, int64_t{1} << 19, 4096, nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_moe_gemm_swiglu(&c, mis, 4, nullptr, (int32_t*)f, f, f, 4, 2, 64, 4096, nullptr), INV_E_ARG);
  EXPECT(inv_swiglu(&c, nullptr, nullptr, 0, 768, nullptr), INV_OK);
  EXPECT(inv_moe_combine(&c, nullptr, nullptr, nullptr, 0, nullptr, 0, 2048, nullptr), INV_OK);
  inv_contract cfp = with(8, 1, INV_FP32);
  EXPECT(inv_lmhead_logprob(&c, f, f, (int32_t*)f, (float*)f, 4, 512, 256, f, 1 << 30, nullptr), INV_E_CONTRACT);
  EXPECT(inv_lmhead_logprob(&cfp, f, f, (int32_t*)f, (float*)f, 4, 262160, 256, f, 1 << 30, nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_lmhead_logprob(&cfp, f, f, (int32_t*)f, (float*)f, 4, 512, 256, f, 256, nullptr), INV_E_WORKSPACE);
  EXPECT(inv_logprob_block16(&cfp, (float*)f, 10, (int32_t*)f, (float*)f, 4, 16, f, 1 << 30, nullptr), INV_E_ARG);
  inv_contract cg = dflt();
  EXPECT(inv_gdn_prefill(&cg, f, f, f, (float*)f, (float*)f, &dummy, 2, 256, 16, 64, f, nullptr, f, 1 << 30,
                         nullptr),
         INV_E_UNSUPPORTED);
  EXPECT(inv_gdn_prefill(&cg, f, f, f, (float*)f, (float*)f, &dummy, 2, 256, 16, 128, f, nullptr, f, 1024, nullptr),
         INV_E_WORKSPACE);
  EXPECT(inv_gdn_decode(&cg, f, f, f, (float*)f, (float*)f, &dummy, 0, 16, 128, f, f, nullptr), INV_OK);
  EXPECT(inv_gdn_decode(&cg, f, f, f, (float*)f, (float*)f, &dummy, 4, 16, 128, f, nullptr, nullptr), INV_E_ARG);
  EXPECT(inv_bench_mfma_loop(-1, 4, nullptr, nullptr, nullptr), INV_E_ARG);
  EXPECT(inv_bench_mfma_loop(0, 4, nullptr, nullptr, nullptr), INV_OK);
}

static std::string hex(const uint8_t d[32]) {
  static const char* h = "0123456789abcdef";
  std::string s;
  for (int i = 0; i < 32; ++i) {
    s += h[d[i] >> 4];
    s += h[d[i] & 15];
  }
  return s;
}

static void sha_and_json() {
  uint8_t d[32];
  EXPECT(inv_sha256("abc", 3, d), INV_OK);
  if (hex(d) != "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad") std::exit(4);
  EXPECT(inv_sha256(nullptr, 0, d), INV_OK);
  if (hex(d) != "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855") std::exit(5);
  // every length across several padding boundaries, in exactly-sized heap buffers
  for (size_t n = 0; n < 300; ++n) {
    std::vector<uint8_t> buf(n ? n : 1, (uint8_t)(n * 7 + 1));
    EXPECT(inv_sha256(buf.data(), n, d), INV_OK);
  }
  std::vector<uint8_t> big(1 << 20, 0x5a);
  EXPECT(inv_sha256(big.data(), big.size(), d), INV_OK);
  EXPECT(inv_sha256(nullptr, 5, d), INV_E_ARG);

  inv_region_contract e[10];
  for (int r = 0; r < 10; ++r) {
    std::memset(&e[r], 0, sizeof(e[r]));
    e[r].region = 10 - r;  // given out of order: written sorted
    inv_contract_default(&e[r].contract);
  }
  e[0].contract.kv_chunk = 64;                   // gdn.core
  e[7].contract.out_dtype = INV_FP32;            // lm_head
  e[1].contract.out_dtype = INV_FP32;            // fused lm head
  e[6].contract.leaves = 64;                     // logprob
  size_t len = 0;
  EXPECT(inv_contract_json(e, 10, nullptr, 0, &len), INV_OK);
  std::vector<char> text(len + 1);
  EXPECT(inv_contract_json(e, 10, text.data(), len, &len), INV_E_ARG);  // no room for the NUL
  EXPECT(inv_contract_json(e, 10, text.data(), len + 1, &len), INV_OK);
  if (std::strlen(text.data()) != len) std::exit(6);
  for (int kind = 1; kind <= 3; ++kind) {
    EXPECT(inv_contract_digest(e, 10, kind, d), INV_OK);
    EXPECT(inv_contract_verify(e, 10, kind, d), INV_OK);
    d[5] ^= 1;
    EXPECT(inv_contract_verify(e, 10, kind, d), INV_E_CONTRACT);
  }
  EXPECT(inv_contract_digest(e, 10, 9, d), INV_E_ARG);
  inv_region_contract dup[2];
  dup[0] = e[0];
  dup[1] = e[0];
  EXPECT(inv_contract_json(dup, 2, nullptr, 0, &len), INV_E_ARG);
  inv_region_contract unk = e[0];
  unk.region = 42;
  EXPECT(inv_contract_json(&unk, 1, nullptr, 0, &len), INV_E_ARG);
  inv_region_contract topo = e[3];
  topo.contract.ranks = 3;
  EXPECT(inv_contract_json(&topo, 1, nullptr, 0, &len), INV_E_TOPOLOGY);
  EXPECT(inv_contract_json(nullptr, 1, nullptr, 0, &len), INV_E_ARG);
  EXPECT(inv_contract_json(e, 0, nullptr, 0, &len), INV_E_ARG);  // a composition has at least one region
  for (size_t cap = 0; cap < 40; ++cap) {  // every short buffer is refused without a write past it
    std::vector<char> small(cap ? cap : 1);
    EXPECT(inv_contract_json(e, 10, small.data(), cap, &len), INV_E_ARG);
  }
}

int main() {
  contracts();
  workspaces();
  entry_points();
  sha_and_json();
  std::printf("host checks passed: %d\n", g_checks);
  return 0;
}
