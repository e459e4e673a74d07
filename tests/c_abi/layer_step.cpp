// A C-ABI caller with no Python or torch in it: reads one layer step's
// inputs from raw files, runs hswd_layer_step through include/hswd.h on the
// GPU, and writes the output and both caches back to raw files.  Test
// infrastructure (tests/test_gpu_c_abi.py drives it and checks the files
// against the oracle).
//
//   layer_step IN_DIR OUT_DIR B H HKV D S DTYPE RING ROT THETA MAX_POS
//
// IN_DIR holds q.bin (float32 [B,H,D]), k.bin and v.bin ([B,HKV,D]),
// gate.bin ([B,H]), pos.bin (int32 [B]), kc.bin and vc.bin (the caches'
// raw bytes, [B,HKV,S,D] of DTYPE, an hswd_dtype code) and, for fp8,
// scale.bin (float32 [2,HKV]).  OUT_DIR receives out.bin, kc.bin and vc.bin.
// Exit status: 0, or 1 with a message on stderr.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/hswd.h"

namespace {

bool read_file(const std::string& path, std::vector<char>& buf, size_t bytes) {
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    buf.resize(bytes);
    const size_t got = bytes ? std::fread(buf.data(), 1, bytes, f) : 0;
    std::fclose(f);
    return got == bytes;
}

bool write_file(const std::string& path, const std::vector<char>& buf) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const size_t put = buf.empty() ? 0 : std::fwrite(buf.data(), 1, buf.size(), f);
    std::fclose(f);
    return put == buf.size();
}

#define CHECK_HIP(x)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

}  // namespace

int main(int argc, char** argv) {
    if (argc != 13) {
        std::fprintf(stderr, "usage: %s IN OUT B H HKV D S DTYPE RING ROT THETA MAX_POS\n", argv[0]);
        return 1;
    }
    const std::string in = argv[1], out = argv[2];
    const int B = std::atoi(argv[3]), H = std::atoi(argv[4]), Hkv = std::atoi(argv[5]);
    const int D = std::atoi(argv[6]), S = std::atoi(argv[7]), dt = std::atoi(argv[8]);
    const int ring = std::atoi(argv[9]), rot = std::atoi(argv[10]);
    const double theta = std::atof(argv[11]);
    const int max_pos = std::atoi(argv[12]);
    const size_t elt = dt == HSWD_F32 ? 4 : (dt == HSWD_FP8_E4M3 ? 1 : 2);
    const size_t cache_bytes = (size_t)B * Hkv * S * D * elt;

    std::vector<char> q, k, v, gate, pos, kc, vc, scale;
    bool ok = read_file(in + "/q.bin", q, (size_t)B * H * D * 4) &&
              read_file(in + "/k.bin", k, (size_t)B * Hkv * D * 4) &&
              read_file(in + "/v.bin", v, (size_t)B * Hkv * D * 4) &&
              read_file(in + "/gate.bin", gate, (size_t)B * H * 4) &&
              read_file(in + "/pos.bin", pos, (size_t)B * 4) &&
              read_file(in + "/kc.bin", kc, cache_bytes) && read_file(in + "/vc.bin", vc, cache_bytes);
    if (ok && dt == HSWD_FP8_E4M3) ok = read_file(in + "/scale.bin", scale, (size_t)2 * Hkv * 4);
    if (!ok) {
        std::fprintf(stderr, "cannot read the inputs in %s\n", in.c_str());
        return 1;
    }

    // device copies (hipMalloc is 256-byte aligned, as the entry points need)
    void *dq, *dk, *dv, *dgate, *dpos, *dkc, *dvc, *dout, *dscale = nullptr, *ws;
    CHECK_HIP(hipMalloc(&dq, q.size()));
    CHECK_HIP(hipMalloc(&dk, k.size()));
    CHECK_HIP(hipMalloc(&dv, v.size()));
    CHECK_HIP(hipMalloc(&dgate, gate.size()));
    CHECK_HIP(hipMalloc(&dpos, pos.size()));
    CHECK_HIP(hipMalloc(&dkc, cache_bytes));
    CHECK_HIP(hipMalloc(&dvc, cache_bytes));
    CHECK_HIP(hipMalloc(&dout, q.size()));
    CHECK_HIP(hipMemcpy(dq, q.data(), q.size(), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, k.data(), k.size(), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v.data(), v.size(), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dgate, gate.data(), gate.size(), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dpos, pos.data(), pos.size(), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dkc, kc.data(), cache_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dvc, vc.data(), cache_bytes, hipMemcpyHostToDevice));
    if (!scale.empty()) {
        CHECK_HIP(hipMalloc(&dscale, scale.size()));
        CHECK_HIP(hipMemcpy(dscale, scale.data(), scale.size(), hipMemcpyHostToDevice));
    }

    hswd_attn_desc d{};
    d.batch = B;
    d.n_heads = H;
    d.n_kv_heads = Hkv;
    d.head_dim = D;
    d.n_slots = S;
    d.kv_dtype = dt;
    d.scale = 1.0f / std::sqrt((float)D);
    d.keys_per_split = 0;
    d.chunks_per_workgroup = 0;
    d.kv_scale = static_cast<const float*>(dscale);

    const size_t ws_bytes = hswd_workspace_bytes(&d, ring, max_pos);
    if (ws_bytes == 0) {
        std::fprintf(stderr, "hswd_workspace_bytes refused the descriptor\n");
        return 1;
    }
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    int32_t st = hswd_workspace_init(ws, ws_bytes, nullptr);
    if (st == HSWD_OK)
        st = hswd_layer_step(static_cast<float*>(dout), static_cast<const float*>(dq),
                             static_cast<const float*>(dk), static_cast<const float*>(dv),
                             static_cast<const float*>(dgate), dkc, dvc,
                             static_cast<const int32_t*>(dpos), ring, rot, theta, max_pos, &d, ws,
                             ws_bytes, nullptr);
    if (st == HSWD_OK) {
        int32_t flags = 0;
        st = hswd_check_errors(ws, &flags, nullptr);
    }
    if (st != HSWD_OK) {
        std::fprintf(stderr, "hswd: %s\n", hswd_status_string(st));
        return 1;
    }

    std::vector<char> o(q.size());
    CHECK_HIP(hipMemcpy(o.data(), dout, o.size(), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(kc.data(), dkc, cache_bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(vc.data(), dvc, cache_bytes, hipMemcpyDeviceToHost));
    if (!(write_file(out + "/out.bin", o) && write_file(out + "/kc.bin", kc) &&
          write_file(out + "/vc.bin", vc))) {
        std::fprintf(stderr, "cannot write the outputs in %s\n", out.c_str());
        return 1;
    }
    for (void* p : {dq, dk, dv, dgate, dpos, dkc, dvc, dout, ws}) CHECK_HIP(hipFree(p));
    if (dscale) CHECK_HIP(hipFree(dscale));
    std::printf("layer_step ok: B=%d H=%d Hkv=%d D=%d S=%d dtype=%d ring=%d\n", B, H, Hkv, D, S, dt,
                ring);
    return 0;
}
