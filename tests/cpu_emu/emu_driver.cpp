// Runs libattn_int8's C ABI on the CPU emulation of HIP (test infrastructure).
// Every "device" buffer is a host allocation of exactly the size the ABI
// documents, so AddressSanitizer reports any access outside it.
//
//   emu_driver quant  x.bin dt n_rows n_cols rps  q.out s.out
//   emu_driver fwd    q.bin sq.bin k.bin sk.bin v.bin sv.bin vmode odt
//                     B H Hkv Lq Lkv d causal  o.out lse.out
//   emu_driver fwdlut q.bin sq.bin k.bin sk.bin v.bin sv.bin vmode odt
//                     B H Hkv Lq Lkv d causal bits clip  o.out lse.out
//   emu_driver lut    bits clip  table.out
//   emu_driver qcols  x.bin dt n_groups rows n_cols  q.out s.out
//   emu_driver q4     x.bin dt n_rows n_cols  codes.out packed.out s.out
//   emu_driver qrot   x.bin dt n_rows n_cols bits  codes.out packed.out s.out
//   emu_driver app4   x.bin dt B Hkv T d L_max pos  cache4.out scales.out
//   emu_driver fwd4   q.bin sq.bin k4.bin sk.bin v.bin sv.bin vmode odt
//                     B H Hkv Lq Lkv d causal  o.out lse.out
//   emu_driver fwdq   qf.bin qdt k.bin sk.bin v.bin sv.bin vmode odt   (fwdqh: Q rotated first)
//                     B H Hkv Lq Lkv d causal  o.out lse.out qhat.out sq.out
//   emu_driver logits q.bin k.bin B H Hkv Lq Lkv d causal  s.out
//   emu_driver append x.bin dt B Hkv T d L_max pos  cache.out scales.out
//                     (cache and scales start filled with 0x63 bytes)
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "attn_int8.h"

namespace {

void* read_file(const char* path, size_t expect) {
  FILE* f = std::fopen(path, "rb");
  if (!f) { std::fprintf(stderr, "cannot open %s\n", path); std::exit(3); }
  void* q = std::malloc(expect ? expect : 1);   // exact size, so ASan sees overruns
  if (std::fread(q, 1, expect, f) != expect) { std::fprintf(stderr, "short read %s\n", path); std::exit(3); }
  std::fclose(f);
  return q;
}

void write_file(const char* path, const void* p, size_t n) {
  FILE* f = std::fopen(path, "wb");
  std::fwrite(p, 1, n, f);
  std::fclose(f);
}

// malloc'd memory is 16-byte aligned on glibc x86-64; the ABI wants 16 bytes
// for tensors, which the exact-size allocation satisfies.
void* alloc(size_t n) { return std::malloc(n ? n : 1); }

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string mode = argv[1];
  attn_status st;
  if (mode == "quant" && argc == 9) {
    const int dt = std::atoi(argv[3]);
    const int64_t n_rows = std::atoll(argv[4]);
    const int32_t n_cols = std::atoi(argv[5]);
    const int64_t rps = std::atoll(argv[6]);
    const size_t esz = dt == ATTN_F16 ? 2 : 4;
    void* x = read_file(argv[2], n_rows * n_cols * esz);
    int8_t* q = static_cast<int8_t*>(alloc(n_rows * n_cols));
    float* s = static_cast<float*>(alloc(sizeof(float) * (n_rows / rps)));
    st = attn_quantize_rows(x, static_cast<attn_dtype>(dt), n_rows, n_cols, rps, q, s, nullptr);
    write_file(argv[7], q, n_rows * n_cols);
    write_file(argv[8], s, sizeof(float) * (n_rows / rps));
  } else if ((mode == "fwd" && argc == 19) || (mode == "fwdlut" && argc == 21)) {
    const bool lut = mode == "fwdlut";
    const int vmode = std::atoi(argv[8]), odt = std::atoi(argv[9]);
    const int B = std::atoi(argv[10]), H = std::atoi(argv[11]), Hkv = std::atoi(argv[12]);
    const int Lq = std::atoi(argv[13]), Lkv = std::atoi(argv[14]), d = std::atoi(argv[15]);
    const int causal = std::atoi(argv[16]);
    const size_t nq = size_t(B) * H * Lq, nk = size_t(B) * Hkv * Lkv;
    auto* q = static_cast<int8_t*>(read_file(argv[2], nq * d));
    auto* sq = static_cast<float*>(read_file(argv[3], nq * 4));
    auto* k = static_cast<int8_t*>(read_file(argv[4], nk * d));
    auto* sk = static_cast<float*>(read_file(argv[5], nk * 4));
    auto* v = static_cast<int8_t*>(read_file(argv[6], nk * d));
    auto* sv = static_cast<float*>(read_file(argv[7], (vmode == 1 ? nk : vmode == 2 ? size_t(B) * Hkv : vmode == 3 ? size_t(B) * Hkv * d : 1) * 4));
    const size_t osz = nq * d * (odt == ATTN_F16 ? 2 : 4);
    void* o = alloc(osz);
    float* lse = static_cast<float*>(alloc(nq * 4));
    const size_t ws_n = attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal);
    void* ws = ws_n ? std::aligned_alloc(256, (ws_n + 255) / 256 * 256) : nullptr;
    if (lut)
      st = attn_int8_fwd_index_softmax(q, sq, k, sk, v, sv, static_cast<attn_vscale>(vmode), o,
                                       static_cast<attn_dtype>(odt), lse, B, H, Hkv, Lq, Lkv, d, causal,
                                       std::atoi(argv[17]), std::strtof(argv[18], nullptr), ws, ws_n,
                                       nullptr);
    else
      st = attn_int8_fwd(q, sq, k, sk, v, sv, static_cast<attn_vscale>(vmode), o,
                         static_cast<attn_dtype>(odt), lse, B, H, Hkv, Lq, Lkv, d, causal, ws, ws_n,
                         nullptr);
    write_file(argv[lut ? 19 : 17], o, osz);
    write_file(argv[lut ? 20 : 18], lse, nq * 4);
  } else if (mode == "qcols" && argc == 9) {
    const int dt = std::atoi(argv[3]);
    const int64_t n_groups = std::atoll(argv[4]), rows = std::atoll(argv[5]);
    const int32_t n_cols = std::atoi(argv[6]);
    const size_t n = size_t(n_groups) * rows * n_cols;
    void* x = read_file(argv[2], n * (dt == ATTN_F16 ? 2 : 4));
    auto* q = static_cast<int8_t*>(alloc(n));
    auto* sc = static_cast<float*>(alloc(size_t(n_groups) * n_cols * 4));
    st = attn_quantize_cols(x, static_cast<attn_dtype>(dt), n_groups, rows, n_cols, q, sc, nullptr);
    write_file(argv[7], q, n);
    write_file(argv[8], sc, size_t(n_groups) * n_cols * 4);
  } else if (mode == "q4" && argc == 9) {
    const int dt = std::atoi(argv[3]);
    const int64_t n_rows = std::atoll(argv[4]);
    const int32_t n_cols = std::atoi(argv[5]);
    const size_t n = size_t(n_rows) * n_cols;
    void* x = read_file(argv[2], n * (dt == ATTN_F16 ? 2 : 4));
    auto* c = static_cast<int8_t*>(alloc(n));
    auto* pk = static_cast<uint8_t*>(alloc(n / 2));
    auto* sc = static_cast<float*>(alloc(size_t(n_rows) * 4));
    st = attn_quantize_rows_int4(x, static_cast<attn_dtype>(dt), n_rows, n_cols, c, pk, sc, nullptr);
    write_file(argv[6], c, n);
    write_file(argv[7], pk, n / 2);
    write_file(argv[8], sc, size_t(n_rows) * 4);
  } else if (mode == "app4" && argc == 12) {
    const int dt = std::atoi(argv[3]);
    const int B = std::atoi(argv[4]), Hkv = std::atoi(argv[5]), T = std::atoi(argv[6]);
    const int d = std::atoi(argv[7]), L = std::atoi(argv[8]), pos = std::atoi(argv[9]);
    void* x = read_file(argv[2], size_t(B) * Hkv * T * d * (dt == ATTN_F16 ? 2 : 4));
    const size_t nc = size_t(B) * Hkv * L * d / 2, ns = size_t(B) * Hkv * L;
    auto* c = static_cast<uint8_t*>(alloc(nc));
    auto* sc = static_cast<float*>(alloc(ns * 4));
    std::memset(c, 0x63, nc);
    std::memset(sc, 0x63, ns * 4);
    st = attn_kv_append_int4(x, static_cast<attn_dtype>(dt), B, Hkv, T, d, c, sc, L, pos, nullptr);
    write_file(argv[10], c, nc);
    write_file(argv[11], sc, ns * 4);
  } else if (mode == "fwd4" && argc == 19) {
    const int vmode = std::atoi(argv[8]), odt = std::atoi(argv[9]);
    const int B = std::atoi(argv[10]), H = std::atoi(argv[11]), Hkv = std::atoi(argv[12]);
    const int Lq = std::atoi(argv[13]), Lkv = std::atoi(argv[14]), d = std::atoi(argv[15]);
    const int causal = std::atoi(argv[16]);
    const size_t nq = size_t(B) * H * Lq, nk = size_t(B) * Hkv * Lkv;
    auto* q = static_cast<int8_t*>(read_file(argv[2], nq * d));
    auto* sq = static_cast<float*>(read_file(argv[3], nq * 4));
    auto* k4 = static_cast<uint8_t*>(read_file(argv[4], nk * d / 2));
    auto* sk = static_cast<float*>(read_file(argv[5], nk * 4));
    auto* v = static_cast<int8_t*>(read_file(argv[6], nk * d));
    auto* sv = static_cast<float*>(read_file(argv[7], (vmode == 1 ? nk : vmode == 2 ? size_t(B) * Hkv : vmode == 3 ? size_t(B) * Hkv * d : 1) * 4));
    const size_t osz = nq * d * (odt == ATTN_F16 ? 2 : 4);
    void* o = alloc(osz);
    float* lse = static_cast<float*>(alloc(nq * 4));
    const size_t ws_n = attn_int4qk_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal);
    void* ws = ws_n ? std::aligned_alloc(256, (ws_n + 255) / 256 * 256) : nullptr;
    st = attn_int4qk_fwd(q, sq, k4, sk, v, sv, static_cast<attn_vscale>(vmode), o, static_cast<attn_dtype>(odt), lse,
                         B, H, Hkv, Lq, Lkv, d, causal, ws, ws_n, nullptr);
    write_file(argv[17], o, osz);
    write_file(argv[18], lse, nq * 4);
  } else if (mode == "qrot" && argc == 10) {
    const int dt = std::atoi(argv[3]);
    const int64_t n_rows = std::atoll(argv[4]);
    const int32_t n_cols = std::atoi(argv[5]);
    const int bits = std::atoi(argv[6]);
    const size_t n = size_t(n_rows) * n_cols;
    void* x = read_file(argv[2], n * (dt == ATTN_F16 ? 2 : 4));
    auto* c = static_cast<int8_t*>(alloc(n));
    auto* pk = static_cast<uint8_t*>(alloc(n / 2));
    auto* sc = static_cast<float*>(alloc(size_t(n_rows) * 4));
    st = attn_quantize_rows_hadamard(x, static_cast<attn_dtype>(dt), n_rows, n_cols, bits, c, bits == 4 ? pk : nullptr,
                                     sc, nullptr);
    write_file(argv[7], c, n);
    write_file(argv[8], pk, n / 2);
    write_file(argv[9], sc, size_t(n_rows) * 4);
  } else if (mode == "lut" && argc == 5) {
    const int bits = std::atoi(argv[2]);
    uint8_t tab[256];
    st = attn_index_softmax_table(bits, std::strtof(argv[3], nullptr), tab);
    write_file(argv[4], tab, bits >= 1 && bits <= 8 ? size_t(1) << bits : 0);
  } else if ((mode == "fwdq" || mode == "fwdqh") && argc == 21) {
    const int qdt = std::atoi(argv[3]);
    const int vmode = std::atoi(argv[8]), odt = std::atoi(argv[9]);
    const int B = std::atoi(argv[10]), H = std::atoi(argv[11]), Hkv = std::atoi(argv[12]);
    const int Lq = std::atoi(argv[13]), Lkv = std::atoi(argv[14]), d = std::atoi(argv[15]);
    const int causal = std::atoi(argv[16]);
    const size_t nq = size_t(B) * H * Lq, nk = size_t(B) * Hkv * Lkv;
    void* qf = read_file(argv[2], nq * d * (qdt == ATTN_F16 ? 2 : 4));
    auto* k = static_cast<int8_t*>(read_file(argv[4], nk * d));
    auto* sk = static_cast<float*>(read_file(argv[5], nk * 4));
    auto* v = static_cast<int8_t*>(read_file(argv[6], nk * d));
    auto* sv = static_cast<float*>(read_file(argv[7], (vmode == 1 ? nk : vmode == 2 ? size_t(B) * Hkv : vmode == 3 ? size_t(B) * Hkv * d : 1) * 4));
    const size_t osz = nq * d * (odt == ATTN_F16 ? 2 : 4);
    void* o = alloc(osz);
    float* lse = static_cast<float*>(alloc(nq * 4));
    auto* qh = static_cast<int8_t*>(alloc(nq * d));
    float* sq = static_cast<float*>(alloc(nq * 4));
    const size_t ws_n = attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal);
    void* ws = ws_n ? std::aligned_alloc(256, (ws_n + 255) / 256 * 256) : nullptr;
    st = (mode == "fwdqh" ? attn_int8_fwd_qfloat_hadamard : attn_int8_fwd_qfloat)(
        qf, static_cast<attn_dtype>(qdt), k, sk, v, sv, static_cast<attn_vscale>(vmode), o,
        static_cast<attn_dtype>(odt), lse, qh, sq, B, H, Hkv, Lq, Lkv, d, causal, ws, ws_n, nullptr);
    write_file(argv[17], o, osz);
    write_file(argv[18], lse, nq * 4);
    write_file(argv[19], qh, nq * d);
    write_file(argv[20], sq, nq * 4);
  } else if (mode == "append" && argc == 12) {
    const int dt = std::atoi(argv[3]);
    const int B = std::atoi(argv[4]), Hkv = std::atoi(argv[5]), T = std::atoi(argv[6]);
    const int d = std::atoi(argv[7]), L = std::atoi(argv[8]), pos = std::atoi(argv[9]);
    const size_t esz = dt == ATTN_F16 ? 2 : 4;
    void* x = read_file(argv[2], size_t(B) * Hkv * T * d * esz);
    const size_t nc = size_t(B) * Hkv * L * d, ns = size_t(B) * Hkv * L;
    auto* c = static_cast<int8_t*>(alloc(nc));
    auto* sc = static_cast<float*>(alloc(ns * 4));
    std::memset(c, 0x63, nc);
    std::memset(sc, 0x63, ns * 4);
    st = attn_kv_append(x, static_cast<attn_dtype>(dt), B, Hkv, T, d, c, sc, L, pos, nullptr);
    write_file(argv[10], c, nc);
    write_file(argv[11], sc, ns * 4);
  } else if (mode == "logits" && argc == 12) {
    const int B = std::atoi(argv[4]), H = std::atoi(argv[5]), Hkv = std::atoi(argv[6]);
    const int Lq = std::atoi(argv[7]), Lkv = std::atoi(argv[8]), d = std::atoi(argv[9]);
    const int causal = std::atoi(argv[10]);
    const size_t nq = size_t(B) * H * Lq, nk = size_t(B) * Hkv * Lkv;
    auto* q = static_cast<int8_t*>(read_file(argv[2], nq * d));
    auto* k = static_cast<int8_t*>(read_file(argv[3], nk * d));
    auto* s = static_cast<int32_t*>(alloc(nq * Lkv * 4));
    for (size_t i = 0; i < nq * Lkv; ++i) s[i] = INT32_MIN;
    st = attn_int8_debug_logits(q, k, B, H, Hkv, Lq, Lkv, d, causal, s, nullptr);
    write_file(argv[11], s, nq * Lkv * 4);
  } else {
    std::fprintf(stderr, "bad arguments\n");
    return 2;
  }
  if (st != ATTN_OK) {
    std::fprintf(stderr, "status %d: %s\n", st, attn_status_str(st));
    return 4;
  }
  return 0;
}
