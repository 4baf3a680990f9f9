// lema_ckpt.cpp -- checkpoint files of include/lema.h (lema_checkpoint_save,
// lema_checkpoint_load).
//
// LEMA README, "Features" (interval-based checkpointing of the full
// fine-tuning delta with the optimizer states) and "Selective Full
// Fine-Tuning" (checkpoints hold the fp32 delta plus the optimizer state and
// are written as safetensors files, which merge_delta reads).  The file is
// safetensors: an 8-byte little-endian header length, a JSON header mapping
// each tensor name to {"dtype", "shape", "data_offsets"} (plus an optional
// "__metadata__" map of strings), then the tensors' bytes back to back.
//
// Data moves between device memory and the file through two page-locked
// staging buffers: while one chunk is being written to (or read from) the
// file, the next one is copied on the caller's stream, so the device copies
// hide behind the file I/O.
#include <fcntl.h>
#include <hip/hip_runtime_api.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <utility>
#include <vector>

#include "lema.h"
#include "lema_host_internal.h"

namespace lema {
namespace {

constexpr size_t kStagingBytes = size_t(64) << 20;     // per staging buffer
constexpr uint64_t kMaxHeaderBytes = uint64_t(100) << 20;
constexpr size_t kMaxName = 255;

const char *dtype_name(int32_t d) {
    switch (d) {
    case LEMA_DT_F32: return "F32";
    case LEMA_DT_BF16: return "BF16";
    case LEMA_DT_I8: return "I8";
    default: return nullptr;
    }
}

size_t dtype_bytes(int32_t d) { return d == LEMA_DT_F32 ? 4 : d == LEMA_DT_BF16 ? 2 : 1; }

// Names are written into the JSON header verbatim, so they are limited to
// printable ASCII that needs no escaping.
bool name_ok(const char *s) {
    const size_t n = strnlen(s, kMaxName + 1);
    if (n == 0 || n > kMaxName) return false;
    for (size_t i = 0; i < n; ++i) {
        const unsigned char c = static_cast<unsigned char>(s[i]);
        if (c < 0x20 || c > 0x7E || c == '"' || c == '\\') return false;
    }
    return true;
}

lema_status validate(const lema_ckpt_tensor *t, int32_t n) {
    if (n < 0) return LEMA_ERR_SIZE;
    if (n > 0 && t == nullptr) return LEMA_ERR_NULL;
    std::vector<std::string> names;
    for (int32_t i = 0; i < n; ++i) {
        if (t[i].name == nullptr) return LEMA_ERR_NULL;
        if (dtype_name(t[i].dtype) == nullptr) return LEMA_ERR_DTYPE;
        if (t[i].numel < 0 || t[i].reserved != 0 || !name_ok(t[i].name)) return LEMA_ERR_SIZE;
        if (t[i].numel > INT64_MAX / 4) return LEMA_ERR_SIZE;
        if (t[i].numel > 0 && t[i].data == nullptr) return LEMA_ERR_NULL;
        names.emplace_back(t[i].name);
    }
    std::sort(names.begin(), names.end());
    if (std::adjacent_find(names.begin(), names.end()) != names.end()) return LEMA_ERR_SIZE;
    return LEMA_OK;
}

// ------------------------------------------------------------ JSON header

// A JSON value of the subset safetensors headers use: objects, arrays,
// strings and integers (true, false and null are accepted and ignored).
struct Json {
    enum Kind { kNull, kInt, kString, kArray, kObject } kind = kNull;
    int64_t i = 0;
    std::string s;
    std::vector<Json> a;
    std::vector<std::pair<std::string, Json>> o;
};

class Parser {
  public:
    Parser(const char *p, size_t n) : p_(p), end_(p + n) {}

    bool document(Json &out) {
        if (!value(out, 0)) return false;
        ws();
        return p_ == end_;
    }

  private:
    const char *p_, *end_;

    void ws() {
        while (p_ < end_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
    }

    bool literal(const char *lit) {
        const size_t n = strlen(lit);
        if (size_t(end_ - p_) < n || memcmp(p_, lit, n) != 0) return false;
        p_ += n;
        return true;
    }

    static void utf8(uint32_t cp, std::string &out) {
        if (cp < 0x80) {
            out += char(cp);
        } else if (cp < 0x800) {
            out += char(0xC0 | (cp >> 6));
            out += char(0x80 | (cp & 0x3F));
        } else if (cp < 0x10000) {
            out += char(0xE0 | (cp >> 12));
            out += char(0x80 | ((cp >> 6) & 0x3F));
            out += char(0x80 | (cp & 0x3F));
        } else {
            out += char(0xF0 | (cp >> 18));
            out += char(0x80 | ((cp >> 12) & 0x3F));
            out += char(0x80 | ((cp >> 6) & 0x3F));
            out += char(0x80 | (cp & 0x3F));
        }
    }

    bool hex4(uint32_t &v) {
        if (end_ - p_ < 4) return false;
        v = 0;
        for (int k = 0; k < 4; ++k) {
            const char c = *p_++;
            v <<= 4;
            if (c >= '0' && c <= '9') v |= uint32_t(c - '0');
            else if (c >= 'a' && c <= 'f') v |= uint32_t(c - 'a' + 10);
            else if (c >= 'A' && c <= 'F') v |= uint32_t(c - 'A' + 10);
            else return false;
        }
        return true;
    }

    bool string(std::string &out) {
        if (p_ >= end_ || *p_ != '"') return false;
        ++p_;
        while (p_ < end_) {
            const unsigned char c = static_cast<unsigned char>(*p_++);
            if (c == '"') return true;
            if (c < 0x20) return false;
            if (c != '\\') {
                out += char(c);
                continue;
            }
            if (p_ >= end_) return false;
            const char e = *p_++;
            switch (e) {
            case '"': out += '"'; break;
            case '\\': out += '\\'; break;
            case '/': out += '/'; break;
            case 'b': out += '\b'; break;
            case 'f': out += '\f'; break;
            case 'n': out += '\n'; break;
            case 'r': out += '\r'; break;
            case 't': out += '\t'; break;
            case 'u': {
                uint32_t cp;
                if (!hex4(cp)) return false;
                if (cp >= 0xD800 && cp < 0xDC00) {          // a surrogate pair
                    uint32_t lo;
                    if (!literal("\\u") || !hex4(lo) || lo < 0xDC00 || lo >= 0xE000) return false;
                    cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
                } else if (cp >= 0xDC00 && cp < 0xE000) {
                    return false;
                }
                utf8(cp, out);
                break;
            }
            default: return false;
            }
        }
        return false;
    }

    // Integers only: safetensors headers hold no fractions or exponents.
    bool integer(int64_t &v) {
        const bool neg = p_ < end_ && *p_ == '-';
        if (neg) ++p_;
        if (p_ >= end_ || *p_ < '0' || *p_ > '9') return false;
        uint64_t u = 0;
        while (p_ < end_ && *p_ >= '0' && *p_ <= '9') {
            const uint64_t d = uint64_t(*p_++ - '0');
            if (u > (uint64_t(INT64_MAX) - d) / 10) return false;
            u = u * 10 + d;
        }
        if (p_ < end_ && (*p_ == '.' || *p_ == 'e' || *p_ == 'E')) return false;
        v = neg ? -int64_t(u) : int64_t(u);
        return true;
    }

    bool value(Json &out, int depth) {
        if (depth > 16) return false;
        ws();
        if (p_ >= end_) return false;
        const char c = *p_;
        if (c == '{') {
            ++p_;
            out.kind = Json::kObject;
            ws();
            if (p_ < end_ && *p_ == '}') {
                ++p_;
                return true;
            }
            for (;;) {
                ws();
                std::string key;
                if (!string(key)) return false;
                ws();
                if (p_ >= end_ || *p_++ != ':') return false;
                Json v;
                if (!value(v, depth + 1)) return false;
                out.o.emplace_back(std::move(key), std::move(v));
                ws();
                if (p_ >= end_) return false;
                if (*p_ == ',') {
                    ++p_;
                    continue;
                }
                if (*p_++ != '}') return false;
                return true;
            }
        }
        if (c == '[') {
            ++p_;
            out.kind = Json::kArray;
            ws();
            if (p_ < end_ && *p_ == ']') {
                ++p_;
                return true;
            }
            for (;;) {
                Json v;
                if (!value(v, depth + 1)) return false;
                out.a.push_back(std::move(v));
                ws();
                if (p_ >= end_) return false;
                if (*p_ == ',') {
                    ++p_;
                    continue;
                }
                if (*p_++ != ']') return false;
                return true;
            }
        }
        if (c == '"') {
            out.kind = Json::kString;
            return string(out.s);
        }
        if (c == '-' || (c >= '0' && c <= '9')) {
            out.kind = Json::kInt;
            return integer(out.i);
        }
        out.kind = Json::kNull;
        return literal("true") || literal("false") || literal("null");
    }
};

const Json *member(const Json &obj, const char *key) {
    for (const auto &kv : obj.o)
        if (kv.first == key) return &kv.second;
    return nullptr;
}

size_t file_dtype_bytes(const std::string &d) {
    static const std::map<std::string, size_t> sizes = {
        {"BOOL", 1}, {"U8", 1},  {"I8", 1},  {"F8_E4M3", 1}, {"F8_E5M2", 1},
        {"I16", 2},  {"U16", 2}, {"F16", 2}, {"BF16", 2},    {"I32", 4},
        {"U32", 4},  {"F32", 4}, {"I64", 8}, {"U64", 8},     {"F64", 8}};
    const auto it = sizes.find(d);
    return it == sizes.end() ? 0 : it->second;
}

struct Entry {
    std::string dtype;
    int64_t numel;
    uint64_t begin, end;    // byte range within the data section
};

// Parses and checks a header: every tensor's shape, dtype and byte range
// must agree and lie inside the data section of `data_bytes`.
lema_status parse_header(const std::string &text, uint64_t data_bytes,
                         std::map<std::string, Entry> &out, int64_t &step) {
    Json root;
    Parser parser(text.data(), text.size());
    if (!parser.document(root) || root.kind != Json::kObject) return LEMA_ERR_IO;
    step = -1;
    for (const auto &kv : root.o) {
        const Json &v = kv.second;
        if (v.kind != Json::kObject) return LEMA_ERR_IO;
        if (kv.first == "__metadata__") {
            // a step that is not an integer (another writer's metadata) reads as -1
            const Json *st = member(v, "step");
            if (st != nullptr && st->kind == Json::kString) {
                Json n;
                Parser p(st->s.data(), st->s.size());
                if (p.document(n) && n.kind == Json::kInt) step = n.i;
            }
            continue;
        }
        const Json *dt = member(v, "dtype"), *shape = member(v, "shape"),
                   *offs = member(v, "data_offsets");
        if (!dt || !shape || !offs || dt->kind != Json::kString || shape->kind != Json::kArray ||
            offs->kind != Json::kArray || offs->a.size() != 2)
            return LEMA_ERR_IO;
        int64_t numel = 1;
        for (const Json &d : shape->a) {
            if (d.kind != Json::kInt || d.i < 0) return LEMA_ERR_IO;
            if (d.i != 0 && numel > INT64_MAX / d.i) return LEMA_ERR_IO;
            numel *= d.i;
        }
        const Json &b = offs->a[0], &e = offs->a[1];
        if (b.kind != Json::kInt || e.kind != Json::kInt || b.i < 0 || e.i < b.i ||
            uint64_t(e.i) > data_bytes)
            return LEMA_ERR_IO;
        const size_t esz = file_dtype_bytes(dt->s);
        if (esz != 0 && (numel > INT64_MAX / int64_t(esz) || e.i - b.i != numel * int64_t(esz)))
            return LEMA_ERR_IO;
        if (!out.emplace(kv.first, Entry{dt->s, numel, uint64_t(b.i), uint64_t(e.i)}).second)
            return LEMA_ERR_IO;     // a name given twice
    }
    return LEMA_OK;
}

// ------------------------------------------------------------- transfers

struct Staging {
    void *buf[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};
    size_t bytes = 0;

    hipError_t init(size_t total) {
        bytes = std::max<size_t>(std::min(kStagingBytes, total), 1);
        for (int k = 0; k < 2; ++k) {
            hipError_t e = hipHostMalloc(&buf[k], bytes, hipHostMallocDefault);
            if (e != hipSuccess) return e;
            e = hipEventCreateWithFlags(&ev[k], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }

    ~Staging() {
        for (int k = 0; k < 2; ++k) {
            if (ev[k]) (void)hipEventDestroy(ev[k]);
            if (buf[k]) (void)hipHostFree(buf[k]);
        }
    }
};

// One piece of the data section: `bytes` at `file_off` (relative to the
// data section) and device address `dev`.
struct Piece {
    uint64_t file_off;
    char *dev;
    size_t bytes;
};

std::vector<Piece> pieces_of(const std::vector<std::pair<uint64_t, const lema_ckpt_tensor *>> &ts,
                             size_t chunk) {
    std::vector<Piece> out;
    for (const auto &ft : ts) {
        const size_t total = size_t(ft.second->numel) * dtype_bytes(ft.second->dtype);
        char *dev = static_cast<char *>(ft.second->data);
        for (size_t o = 0; o < total; o += chunk)
            out.push_back({ft.first + o, dev + o, std::min(chunk, total - o)});
    }
    return out;
}

bool write_all(int fd, const char *p, size_t n) {
    while (n > 0) {
        const ssize_t w = ::write(fd, p, n);
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        p += w;
        n -= size_t(w);
    }
    return true;
}

bool read_all(int fd, char *p, size_t n, uint64_t off) {
    while (n > 0) {
        const ssize_t r = ::pread(fd, p, n, off_t(off));
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        p += r;
        n -= size_t(r);
        off += uint64_t(r);
    }
    return true;
}

lema_status capture_check(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_failed(e);
    return cs == hipStreamCaptureStatusNone ? LEMA_OK : LEMA_ERR_CAPTURE;
}

// Closes the file descriptor on scope exit and removes the temporary file
// unless `keep` is set.
struct TmpFile {
    int fd = -1;
    std::string path;
    bool keep = false;
    ~TmpFile() {
        if (fd >= 0) ::close(fd);
        if (!keep && !path.empty()) ::unlink(path.c_str());
    }
};

struct InFile {
    int fd = -1;
    ~InFile() {
        if (fd >= 0) ::close(fd);
    }
};

}  // namespace
}  // namespace lema

using namespace lema;

extern "C" {

lema_status lema_checkpoint_save(const char *path, const lema_ckpt_tensor *t, int32_t n,
                                 int64_t step, void *stream) {
    if (path == nullptr) return LEMA_ERR_NULL;
    lema_status st = validate(t, n);
    if (st != LEMA_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);

    // header: tensors in the order given, back to back
    std::string h = "{\"__metadata__\":{\"format\":\"lema-checkpoint\",\"step\":\"" +
                    std::to_string(step) + "\"}";
    std::vector<std::pair<uint64_t, const lema_ckpt_tensor *>> order;
    uint64_t off = 0;
    for (int32_t i = 0; i < n; ++i) {
        const uint64_t bytes = uint64_t(t[i].numel) * dtype_bytes(t[i].dtype);
        h += ",\"" + std::string(t[i].name) + "\":{\"dtype\":\"" + dtype_name(t[i].dtype) +
             "\",\"shape\":[" + std::to_string(t[i].numel) + "],\"data_offsets\":[" +
             std::to_string(off) + "," + std::to_string(off + bytes) + "]}";
        order.emplace_back(off, &t[i]);
        off += bytes;
    }
    h += "}";
    while (h.size() % 8 != 0) h += ' ';

    Staging stg;
    hipError_t e = hipSuccess;
    if (off > 0) {          // device copies only when some tensor holds data
        st = capture_check(hs);
        if (st != LEMA_OK) return st;
        if ((e = stg.init(size_t(off))) != hipSuccess) return hip_failed(e);
    }

    // a temporary file of its own next to `path` (concurrent saves to one
    // path do not share it), renamed over `path` once complete
    TmpFile tmp;
    std::string name = std::string(path) + ".tmp.XXXXXX";
    tmp.fd = ::mkostemp(&name[0], O_CLOEXEC);
    if (tmp.fd < 0) return LEMA_ERR_IO;
    tmp.path = name;
    if (::fchmod(tmp.fd, 0644) != 0) return LEMA_ERR_IO;
    unsigned char len[8];
    for (int k = 0; k < 8; ++k) len[k] = static_cast<unsigned char>(uint64_t(h.size()) >> (8 * k));
    if (!write_all(tmp.fd, reinterpret_cast<const char *>(len), 8) ||
        !write_all(tmp.fd, h.data(), h.size()))
        return LEMA_ERR_IO;

    // device -> staging[k % 2] on the stream, then staging -> file, with the
    // next piece's copy in flight while this one is written
    const std::vector<Piece> ps = pieces_of(order, stg.bytes);
    auto issue = [&](size_t k) -> hipError_t {
        const int b = int(k % 2);
        hipError_t err = hipMemcpyAsync(stg.buf[b], ps[k].dev, ps[k].bytes, hipMemcpyDefault, hs);
        return err != hipSuccess ? err : hipEventRecord(stg.ev[b], hs);
    };
    if (!ps.empty() && (e = issue(0)) != hipSuccess) return hip_failed(e);
    for (size_t k = 0; k < ps.size(); ++k) {
        if (k + 1 < ps.size() && (e = issue(k + 1)) != hipSuccess) {
            (void)hipStreamSynchronize(hs);
            return hip_failed(e);
        }
        if ((e = hipEventSynchronize(stg.ev[k % 2])) != hipSuccess) {
            (void)hipStreamSynchronize(hs);
            return hip_failed(e);
        }
        if (!write_all(tmp.fd, static_cast<const char *>(stg.buf[k % 2]), ps[k].bytes)) {
            (void)hipStreamSynchronize(hs);
            return LEMA_ERR_IO;
        }
    }
    if (off > 0 && (e = hipStreamSynchronize(hs)) != hipSuccess) return hip_failed(e);
    if (::fsync(tmp.fd) != 0) return LEMA_ERR_IO;
    const int fd = tmp.fd;
    tmp.fd = -1;
    if (::close(fd) != 0) return LEMA_ERR_IO;
    if (::rename(tmp.path.c_str(), path) != 0) return LEMA_ERR_IO;
    tmp.keep = true;
    return LEMA_OK;
}

lema_status lema_checkpoint_load(const char *path, const lema_ckpt_tensor *t, int32_t n,
                                 int64_t *step, void *stream) {
    if (path == nullptr) return LEMA_ERR_NULL;
    lema_status st = validate(t, n);
    if (st != LEMA_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);

    InFile in;
    in.fd = ::open(path, O_RDONLY | O_CLOEXEC);
    if (in.fd < 0) return LEMA_ERR_IO;
    struct stat sb;
    if (::fstat(in.fd, &sb) != 0 || sb.st_size < 8) return LEMA_ERR_IO;
    const uint64_t file_bytes = uint64_t(sb.st_size);
    unsigned char len[8];
    if (!read_all(in.fd, reinterpret_cast<char *>(len), 8, 0)) return LEMA_ERR_IO;
    uint64_t hlen = 0;
    for (int k = 0; k < 8; ++k) hlen |= uint64_t(len[k]) << (8 * k);
    if (hlen < 2 || hlen > kMaxHeaderBytes || hlen > file_bytes - 8) return LEMA_ERR_IO;
    std::string text(size_t(hlen), '\0');
    if (!read_all(in.fd, &text[0], size_t(hlen), 8)) return LEMA_ERR_IO;
    const uint64_t data0 = 8 + hlen;
    std::map<std::string, Entry> entries;
    int64_t file_step = -1;
    st = parse_header(text, file_bytes - data0, entries, file_step);
    if (st != LEMA_OK) return st;

    // match every request before touching device memory
    std::vector<std::pair<uint64_t, const lema_ckpt_tensor *>> order;
    uint64_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        const auto it = entries.find(t[i].name);
        if (it == entries.end()) return LEMA_ERR_NOT_FOUND;
        if (it->second.dtype != dtype_name(t[i].dtype)) return LEMA_ERR_DTYPE;
        if (it->second.numel != t[i].numel) return LEMA_ERR_SIZE;
        order.emplace_back(it->second.begin, &t[i]);
        total += it->second.end - it->second.begin;
    }
    if (step != nullptr) *step = file_step;
    if (total == 0) return LEMA_OK;     // nothing to copy (no request, or empty tensors)

    st = capture_check(hs);
    if (st != LEMA_OK) return st;
    Staging stg;
    hipError_t e = stg.init(size_t(total));
    if (e != hipSuccess) return hip_failed(e);

    // file -> staging[k % 2], then staging -> device on the stream; a staging
    // buffer is refilled only after its previous copy has completed
    const std::vector<Piece> ps = pieces_of(order, stg.bytes);
    for (size_t k = 0; k < ps.size(); ++k) {
        const int b = int(k % 2);
        if (k >= 2 && (e = hipEventSynchronize(stg.ev[b])) != hipSuccess) {
            (void)hipStreamSynchronize(hs);
            return hip_failed(e);
        }
        if (!read_all(in.fd, static_cast<char *>(stg.buf[b]), ps[k].bytes,
                      data0 + ps[k].file_off)) {
            (void)hipStreamSynchronize(hs);
            return LEMA_ERR_IO;
        }
        e = hipMemcpyAsync(ps[k].dev, stg.buf[b], ps[k].bytes, hipMemcpyDefault, hs);
        if (e == hipSuccess) e = hipEventRecord(stg.ev[b], hs);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(hs);
            return hip_failed(e);
        }
    }
    if ((e = hipStreamSynchronize(hs)) != hipSuccess) return hip_failed(e);
    return LEMA_OK;
}

}  // extern "C"
