"""Writes pipespec_formulas.txt: the PipeSpec review's closed forms evaluated on
a grid of (alpha, gamma).  Formulas as stated on the PipeSpec review page
("What carries the argument"; "Core claim"; "Assumptions & free parameters").
Run from the repository root: python tests/golden/make_pipespec_formulas.py
"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    rows = []
    for gamma in (1, 4, 8):
        for alpha in (0.05, 0.3, 0.6, 0.9):
            E = (1 - alpha ** (gamma + 1)) / (1 - alpha)
            rho = alpha / (1 - alpha ** (gamma + 1) + alpha)
            EN = (1 - rho) + rho * E
            rows.append(f"{alpha:.2f} {gamma:d} {E:.12f} {rho:.12f} {EN:.12f}")
    with open(os.path.join(HERE, "pipespec_formulas.txt"), "w") as f:
        f.write("# PipeSpec review (pith.science/paper/2505.01572): closed forms on a grid.\n")
        f.write("# E = (1-a^(g+1))/(1-a) tokens per window; rho = a/(1-a^(g+1)+a) steady-state\n")
        f.write("# verification probability; EN = (1-rho) + rho*E expected tokens per step.\n")
        f.write("# alpha gamma E rho EN\n")
        f.write("\n".join(rows) + "\n")


if __name__ == "__main__":
    main()
